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

#include <type_traits>

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
constexpr int UP_LIST = 256;    // entries per wave list (tiles per group * cap)
constexpr int DOWN_LIST = 512;  // entries per wave list (tiles per fill * cap)

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
// Sparse up projection.  NC = 16-byte chunks per lane covering d; U = entries
// in flight per wave (U * NC 16-byte loads per lane outstanding).

template <Dt D, int NC, int U>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_up(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wu,
    const uint16_t *__restrict__ cnt, const typename DtT<D>::T *__restrict__ val,
    const uint8_t *__restrict__ idx, const uint8_t *__restrict__ row_flag, float *__restrict__ vbuf, int T,
    int d, int nt, int tile, int cap, int tpg, int n_groups, int tok_per_wg, int n_tb) {
  using TT = typename DtT<D>::T;
  constexpr int EPC = 16 / sizeof(TT);  // elements per 16-byte chunk
  __shared__ Entry list[SP_WAVES][UP_LIST];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int g, tb;
  group_coords(blockIdx.x, n_groups, n_tb, g, tb);
  const int k0 = g * tpg;
  const int kn = min(tpg, nt - k0);
  Entry *L = list[wave];
  const char *wub = reinterpret_cast<const char *>(wu);
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);

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

    for (int e = 0; e < E; e += U) {
      Entry en[U];
      u32x4_t w[U][NC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        en[u] = L[min(e + u, E - 1)];
        const char *r = wub + (size_t)((uint32_t)(en[u].j & 0x3FFFFFF) * row_bytes) + lane * 16;
#pragma unroll
        for (int c = 0; c < NC; ++c) w[u][c] = *reinterpret_cast<const u32x4_t *>(r + c * 1024);
      }
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) p[u] = dot16(xr[c], w[u][c], p[u], TT());
        p[u] = wave_sum_to_lane63(p[u]);
      }
      if (lane == 63) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (e + u < E) {
            const int j = en[u].j & 0x3FFFFFF, s = (unsigned)en[u].j >> 26;
            vbuf[((size_t)t * nt + j / tile) * cap + s] = en[u].w * p[u];
          }
        }
      }
    }
    wave_sync_lds();
  }
}

// ---------------------------------------------------------------------------
// Sparse down projection.  VPL = output columns per lane (slice = 64 * VPL);
// U = W_d row segments in flight per wave.

template <Dt D, int VPL, int U>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_down(
    const float *__restrict__ vbuf, const uint16_t *__restrict__ cnt, const uint8_t *__restrict__ idx,
    const uint8_t *__restrict__ row_flag, const typename DtT<D>::T *__restrict__ wd,
    typename DtT<D>::T *__restrict__ y, int T, int d, int nt, int tile, int cap, int n_slices, int tok_per_wg,
    int n_tb) {
  using TT = typename DtT<D>::T;
  constexpr int VB = VPL * sizeof(TT);  // bytes per lane per row
  static_assert(VB == 4 || VB == 8 || VB == 16, "lane vector must be 4, 8 or 16 bytes");
  using V = typename std::conditional<VB == 16, u32x4_t,
                                      typename std::conditional<VB == 8, u32x2_t, uint32_t>::type>::type;
  __shared__ Entry list[SP_WAVES][DOWN_LIST];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int sl, tb;
  group_coords(blockIdx.x, n_slices, n_tb, sl, tb);
  const int c0 = sl * 64 * VPL + lane * VPL;
  // lane's column segment of every W_d row: base + row_offset(j) (32-bit)
  const char *wdb = reinterpret_cast<const char *>(wd + c0);
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);
  Entry *L = list[wave];
  const int tiles_per_fill = min(64, DOWN_LIST / cap);

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
        L[o].j = (int)((uint32_t)(k * tile + idx[slot0 + s]) * row_bytes);  // byte offset of the row
        L[o].w = vbuf[slot0 + s];
      }
      wave_sync_lds();
      for (int e = 0; e < E; e += U) {
        Entry en[U];
        V w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          en[u] = L[min(e + u, E - 1)];
          if (e + u >= E) en[u].w = 0.f;  // tail: duplicate row, zero weight
          w[u] = *reinterpret_cast<const V *>(wdb + (uint32_t)en[u].j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t *wv = reinterpret_cast<const uint32_t *>(&w[u]);
          if constexpr (D == Dt::BF16) {
#pragma unroll
            for (int v = 0; v < VPL / 2; ++v) {
              acc[2 * v] = fmaf(en[u].w, bf16lo(wv[v]), acc[2 * v]);
              acc[2 * v + 1] = fmaf(en[u].w, bf16hi(wv[v]), acc[2 * v + 1]);
            }
          } else {
#pragma unroll
            for (int v = 0; v < VPL; ++v) acc[v] = fmaf(en[u].w, __uint_as_float(wv[v]), acc[v]);
          }
        }
      }
      wave_sync_lds();
    }

    V out;
    uint32_t *ov = reinterpret_cast<uint32_t *>(&out);
    if constexpr (D == Dt::BF16) {
#pragma unroll
      for (int v = 0; v < VPL / 2; ++v)
        ov[v] = (uint32_t)bf16_rne(acc[2 * v]) | ((uint32_t)bf16_rne(acc[2 * v + 1]) << 16);
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) ov[v] = __float_as_uint(acc[v]);
    }
    *reinterpret_cast<V *>(y + (size_t)t * d + c0) = out;
  }
}

// ---------------------------------------------------------------------------
// Launchers.

template <Dt D, int NC>
static hipError_t launch_up(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int nt = a.F / a.tile;
  // Tiles per group: about 4 MB of W_u^T rows per group (one XCD's L2); at
  // the 1.5B-class and larger layer shapes this was the fastest setting of a
  // sweep over 1..8 tiles per group.
  const size_t group_target = (size_t)4 << 20;
  const size_t tile_bytes = (size_t)a.tile * a.d * sizeof(TT);
  int tpg = (int)std::max<size_t>(1, group_target / tile_bytes);
  tpg = std::min(tpg, std::min(std::min(64, nt), UP_LIST / a.cap));
  while (nt % tpg != 0) --tpg;
  const int n_groups = nt / tpg;
  const int tok = 16;
  const int n_tb = (a.T + tok - 1) / tok;
  constexpr int U = NC >= 8 ? 2 : 4;
  hipLaunchKernelGGL((k_sparse_up<D, NC, U>), dim3(n_groups * n_tb), dim3(SP_THREADS), 0, s, (const TT *)a.x,
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
  const int tok = 16;
  const int n_tb = (a.T + tok - 1) / tok;
  hipLaunchKernelGGL((k_sparse_down<D, VPL, 8>), dim3(n_slices * n_tb), dim3(SP_THREADS), 0, s, a.vbuf, a.cnt,
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
