// Overflow scan and the sparse up / down projections over TwELL entries.
//
// The inference route of gist.science "Sparser, Faster, Lighter Transformer
// Language Models", Resumen Técnico §2.B: the up and down projections are
// evaluated only for the active gate units read from TwELL.  On MI355X the two
// projections are separate kernels so that each one can keep its own slice of
// weights resident in one XCD's 4 MB L2:
//   up:   hidden units are split into groups of TwELL tiles and group g runs on
//         XCD g % 8; per active entry (t, j) one wave dots x_t (held in
//         registers) with the W_u^T row j, and stores v = h * u in fp32.
//   down: the d output columns are split into slices and slice s runs on
//         XCD s % 8; per token one wave accumulates v * W_d[j][slice] over all
//         the token's entries in fp32 registers and rounds y once.
// Rows flagged by the overflow scan are left to the dense fallback.
#include "launch.hpp"

namespace twell {

// ---------------------------------------------------------------------------
// Overflow scan: row t overflows iff max_k cnt[t][k] > cap.  One workgroup;
// rows are visited in ascending order so the list is deterministic.
constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_ROWS = 4;  // rows in flight per thread

__global__ __launch_bounds__(SCAN_THREADS) void k_overflow_scan(const uint16_t *__restrict__ cnt, int T, int nt,
                                                               int cap, uint8_t *__restrict__ row_flag,
                                                               int *__restrict__ ovf_rows, int ovf_cap,
                                                               int *__restrict__ n_ovf) {
  __shared__ int wcount[SCAN_ROWS][SCAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool vec = (nt % 8) == 0;
  int carry = 0;
  for (int base = 0; base < T; base += SCAN_THREADS * SCAN_ROWS) {
    bool f[SCAN_ROWS];
#pragma unroll
    for (int q = 0; q < SCAN_ROWS; ++q) {
      const int t = base + q * SCAN_THREADS + tid;
      int mx = 0;
      if (t < T) {
        const uint16_t *c = cnt + (size_t)t * nt;
        if (vec) {
          for (int k = 0; k < nt; k += 8) {
            u32x4_t w = *reinterpret_cast<const u32x4_t *>(c + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = max(mx, (int)max(w[e] & 0xFFFFu, w[e] >> 16));
          }
        } else {
          for (int k = 0; k < nt; ++k) mx = max(mx, (int)c[k]);
        }
      }
      f[q] = t < T && mx > cap;
      if (t < T && row_flag != nullptr) row_flag[t] = f[q] ? 1 : 0;
    }
    uint64_t m[SCAN_ROWS];
#pragma unroll
    for (int q = 0; q < SCAN_ROWS; ++q) {
      m[q] = ballot(f[q]);
      if (lane == 0) wcount[q][wave] = popc64(m[q]);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < SCAN_ROWS; ++q) {
      int before = carry;
      for (int w = 0; w < SCAN_THREADS / 64; ++w) before += (w < wave) ? wcount[q][w] : 0;
      if (f[q]) {
        const int pos = before + mbcnt(m[q]);
        if (pos < ovf_cap) ovf_rows[pos] = base + q * SCAN_THREADS + tid;
      }
      for (int w = 0; w < SCAN_THREADS / 64; ++w) carry += wcount[q][w];
    }
    __syncthreads();
  }
  if (tid == 0) *n_ovf = carry;
}

hipError_t overflow_scan(const ScanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_overflow_scan, dim3(1), dim3(SCAN_THREADS), 0, s, a.cnt, a.T, a.nt, a.cap, a.row_flag,
                     a.ovf_rows, a.ovf_cap, a.n_ovf);
  return hipGetLastError();
}

__global__ void k_zero_int(int *p) { *p = 0; }
hipError_t zero_int(int *p, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_int, dim3(1), dim3(1), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared pieces of the up / down kernels.

constexpr int SP_THREADS = 256;
constexpr int SP_WAVES = SP_THREADS / 64;
constexpr int LIST_MAX = 1024;  // entries per wave list

// Block -> (group, token block) so that group g runs on XCD g % 8 when the
// group count is a multiple of 8 (groups beyond 8 run in successive phases).
__device__ __forceinline__ void group_coords(int bid, int n_groups, int n_tb, int &g, int &tb) {
  if (n_groups % 8 == 0) {
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

struct Entry {
  int j;      // hidden unit (global column); bits 26.. hold the slot s for the up kernel
  float w;    // h (up) or v = h*u (down)
};

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

// ---------------------------------------------------------------------------
// Sparse up projection.  NC = 16-byte chunks per lane covering d.

template <Dt D, int NC>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_up(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wu,
    const uint16_t *__restrict__ cnt, const typename DtT<D>::T *__restrict__ val,
    const uint8_t *__restrict__ idx, const uint8_t *__restrict__ row_flag, float *__restrict__ vbuf, int T,
    int d, int nt, int tile, int cap, int tpg, int n_groups, int tok_per_wg, int n_tb) {
  using TT = typename DtT<D>::T;
  constexpr int EPC = 16 / sizeof(TT);  // elements per 16-byte chunk
  __shared__ Entry list[SP_WAVES][LIST_MAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int g, tb;
  group_coords(blockIdx.x, n_groups, n_tb, g, tb);
  const int k0 = g * tpg;
  const int kn = min(tpg, nt - k0);
  Entry *L = list[wave];

  for (int it = wave; it < tok_per_wg; it += SP_WAVES) {
    const int t = tb * tok_per_wg + it;
    if (t >= T) break;
    if (row_flag[t]) continue;
    const TT *xt = x + (size_t)t * d;
    u32x4_t xr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xr[c] = *reinterpret_cast<const u32x4_t *>(xt + (c * 64 + lane) * EPC);

    // Gather the entries of the group's tiles into the wave list (tpg <= 64).
    const int k = k0 + lane;
    const int n = lane < kn ? min((int)cnt[(size_t)t * nt + k], cap) : 0;
    const int incl = wave_incl_scan(n);
    const int E = __shfl(incl, 63, 64);
    const size_t slot0 = ((size_t)t * nt + k) * cap;
    for (int s = 0, o = incl - n; s < n; ++s, ++o) {
      L[o].j = (k * tile + idx[slot0 + s]) | (s << 26);
      L[o].w = to_f32(val[slot0 + s]);
    }
    wave_sync_lds();

    for (int e = 0; e < E; e += 2) {
      const Entry e0 = L[e];
      const bool two = e + 1 < E;
      const Entry e1 = two ? L[e + 1] : e0;
      const int j0 = e0.j & 0x3FFFFFF, j1 = e1.j & 0x3FFFFFF;
      const TT *r0 = wu + (size_t)j0 * d, *r1 = wu + (size_t)j1 * d;
      u32x4_t w0[NC], w1[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        w0[c] = *reinterpret_cast<const u32x4_t *>(r0 + (c * 64 + lane) * EPC);
        w1[c] = *reinterpret_cast<const u32x4_t *>(r1 + (c * 64 + lane) * EPC);
      }
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        p0 = dot16(xr[c], w0[c], p0, TT());
        p1 = dot16(xr[c], w1[c], p1, TT());
      }
      p0 = wave_sum(p0);
      p1 = wave_sum(p1);
      if (lane == 0) {
        const int s0 = (unsigned)e0.j >> 26, s1 = (unsigned)e1.j >> 26;
        vbuf[((size_t)t * nt + j0 / tile) * cap + s0] = e0.w * p0;
        if (two) vbuf[((size_t)t * nt + j1 / tile) * cap + s1] = e1.w * p1;
      }
    }
    wave_sync_lds();
  }
}

// ---------------------------------------------------------------------------
// Sparse down projection.  VPL = output columns per lane (slice = 64 * VPL).

template <Dt D, int VPL>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_down(
    const float *__restrict__ vbuf, const uint16_t *__restrict__ cnt, const uint8_t *__restrict__ idx,
    const uint8_t *__restrict__ row_flag, const typename DtT<D>::T *__restrict__ wd,
    typename DtT<D>::T *__restrict__ y, int T, int d, int nt, int tile, int cap, int n_slices, int tok_per_wg,
    int n_tb) {
  using TT = typename DtT<D>::T;
  constexpr int VB = VPL * sizeof(TT);  // bytes per lane per row
  static_assert(VB == 8 || VB == 16, "lane vector must be 8 or 16 bytes");
  __shared__ Entry list[SP_WAVES][LIST_MAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int sl, tb;
  group_coords(blockIdx.x, n_slices, n_tb, sl, tb);
  const int c0 = sl * 64 * VPL + lane * VPL;
  Entry *L = list[wave];
  const int tiles_per_fill = min(64, LIST_MAX / cap);

  for (int it = wave; it < tok_per_wg; it += SP_WAVES) {
    const int t = tb * tok_per_wg + it;
    if (t >= T) break;
    if (row_flag[t]) continue;
    float acc[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] = 0.f;

    for (int kb = 0; kb < nt; kb += tiles_per_fill) {
      const int k = kb + lane;
      const int n = (lane < tiles_per_fill && k < nt) ? min((int)cnt[(size_t)t * nt + k], cap) : 0;
      const int incl = wave_incl_scan(n);
      const int E = __shfl(incl, 63, 64);
      const size_t slot0 = ((size_t)t * nt + k) * cap;
      for (int s = 0, o = incl - n; s < n; ++s, ++o) {
        L[o].j = k * tile + idx[slot0 + s];
        L[o].w = vbuf[slot0 + s];
      }
      wave_sync_lds();
      int e = 0;
      for (; e + 4 <= E; e += 4) {
        Entry en[4];
        u32x4_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          en[u] = L[e + u];
          const char *p = reinterpret_cast<const char *>(wd + (size_t)en[u].j * d + c0);
          if constexpr (VB == 16) {
            w[u] = *reinterpret_cast<const u32x4_t *>(p);
          } else {
            u32x2_t q = *reinterpret_cast<const u32x2_t *>(p);
            w[u] = u32x4_t{q.x, q.y, 0u, 0u};
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (D == Dt::BF16) {
#pragma unroll
            for (int v = 0; v < VPL / 2; ++v) {
              acc[2 * v] = fmaf(en[u].w, bf16lo(w[u][v]), acc[2 * v]);
              acc[2 * v + 1] = fmaf(en[u].w, bf16hi(w[u][v]), acc[2 * v + 1]);
            }
          } else {
#pragma unroll
            for (int v = 0; v < VPL; ++v) acc[v] = fmaf(en[u].w, __uint_as_float(w[u][v]), acc[v]);
          }
        }
      }
      for (; e < E; ++e) {
        const Entry en = L[e];
        const TT *p = wd + (size_t)en.j * d + c0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[v] = fmaf(en.w, to_f32(p[v]), acc[v]);
      }
      wave_sync_lds();
    }

    TT *yo = y + (size_t)t * d + c0;
    if constexpr (D == Dt::BF16) {
      uint32_t packed[VPL / 2];
#pragma unroll
      for (int v = 0; v < VPL / 2; ++v)
        packed[v] = (uint32_t)bf16_rne(acc[2 * v]) | ((uint32_t)bf16_rne(acc[2 * v + 1]) << 16);
      if constexpr (VB == 16)
        *reinterpret_cast<u32x4_t *>(yo) = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
      else
        *reinterpret_cast<u32x2_t *>(yo) = u32x2_t{packed[0], packed[1]};
    } else {
      if constexpr (VB == 16)
        *reinterpret_cast<f32x4_t *>(yo) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      else
        *reinterpret_cast<f32x2_t *>(yo) = f32x2_t{acc[0], acc[1]};
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.

template <Dt D, int NC>
static hipError_t launch_up(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int nt = a.F / a.tile;
  // Tiles per group: one group per XCD when the tile count allows it, so that
  // each XCD's L2 holds one slice of W_u^T rows.
  int tpg = std::max(1, nt / 8);
  tpg = std::min(tpg, std::min(64, LIST_MAX / a.cap));
  while (nt % tpg != 0) --tpg;
  const int n_groups = nt / tpg;
  const int tok = 32;
  const int n_tb = (a.T + tok - 1) / tok;
  hipLaunchKernelGGL((k_sparse_up<D, NC>), dim3(n_groups * n_tb), dim3(SP_THREADS), 0, s, (const TT *)a.x,
                     (const TT *)a.wu, a.cnt, (const TT *)a.val, a.idx, a.row_flag, a.vbuf, a.T, a.d, nt, a.tile,
                     a.cap, tpg, n_groups, tok, n_tb);
  return hipGetLastError();
}

template <Dt D>
static hipError_t up_dispatch(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int nc = a.d / (64 * (16 / (int)sizeof(TT)));
  switch (nc) {
#define TWELL_UP_CASE(N) \
  case N:                \
    return launch_up<D, N>(a, s);
    TWELL_UP_CASE(1) TWELL_UP_CASE(2) TWELL_UP_CASE(3) TWELL_UP_CASE(4) TWELL_UP_CASE(5) TWELL_UP_CASE(6)
    TWELL_UP_CASE(7) TWELL_UP_CASE(8) TWELL_UP_CASE(9) TWELL_UP_CASE(10) TWELL_UP_CASE(11) TWELL_UP_CASE(12)
    TWELL_UP_CASE(13) TWELL_UP_CASE(14) TWELL_UP_CASE(15) TWELL_UP_CASE(16)
#undef TWELL_UP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t sparse_up(const SparseArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? up_dispatch<Dt::BF16>(a, s) : up_dispatch<Dt::F32>(a, s);
}

template <Dt D, int VPL>
static hipError_t launch_down(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int nt = a.F / a.tile;
  const int n_slices = a.d / (64 * VPL);
  const int tok = 32;
  const int n_tb = (a.T + tok - 1) / tok;
  hipLaunchKernelGGL((k_sparse_down<D, VPL>), dim3(n_slices * n_tb), dim3(SP_THREADS), 0, s, a.vbuf, a.cnt,
                     a.idx, a.row_flag, (const TT *)a.wd, (TT *)a.y, a.T, a.d, nt, a.tile, a.cap, n_slices, tok,
                     n_tb);
  return hipGetLastError();
}

hipError_t sparse_down(const SparseArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  // 256-column slices: VPL 4 (8-byte bf16 / 16-byte fp32 lane vectors).
  return a.dtype == Dt::BF16 ? launch_down<Dt::BF16, 4>(a, s) : launch_down<Dt::F32, 4>(a, s);
}

}  // namespace twell
