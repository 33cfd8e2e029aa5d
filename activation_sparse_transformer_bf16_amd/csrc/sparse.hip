// Overflow scan and the sparse up / down projections over TwELL entries.
//
// The inference route of gist.science "Sparser, Faster, Lighter Transformer
// Language Models", Resumen Técnico §2.B: the up and down projections are
// evaluated only for the active gate units read from TwELL.  On MI355X the two
// projections are separate kernels so that each one can keep its own slice of
// weights resident in one XCD's 4 MB L2:
//   up:   hidden units are split into groups of TwELL tiles and group g runs on
//         XCD g % 8; per active entry (t, j) one wave dots x_t (held in
//         registers) with the W_u^T row j, and writes (row offset of j,
//         v = h * u rounded to the storage dtype) to row t's compact entry
//         list.  v is the down projection's input activation, rounded as the
//         dense layer and the dense fallback round it.
//   down: the d output columns are split into slices and slice s runs on
//         XCD s % 8; per token one wave copies the token's entry list to LDS
//         64 entries at a time, accumulates v * W_d[j][slice] in fp32
//         registers (for bf16: the same columns of two entries interleaved
//         with v_perm, one v_dot2_f32_bf16 per column and entry pair) and
//         rounds y once.
// The up kernel also decides which rows overflow (a tile with more than cap
// entries); those rows are left to the dense fallback.
#include "gather.hpp"
#include "launch.hpp"

#include <algorithm>
#include <type_traits>

namespace twell {

// ---------------------------------------------------------------------------
// Overflow scan: row t overflows iff max_k cnt[t][k] > cap.  One workgroup.
// Rows are taken SCAN_CHUNK at a time: the chunk's counts are read as flat
// streams of 16-byte loads (consecutive threads, consecutive bytes; one stream
// in the row-major layout, one per tile in the tile-major one), a count above
// cap sets its row's flag byte in LDS, and the flags are then compacted in
// ascending row order, so the list is deterministic.
constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_PER = 8;                         // flag bytes per thread in the compaction
constexpr int SCAN_CHUNK = SCAN_PER * SCAN_THREADS;  // rows per round
constexpr int SCAN_LOADS = 16;                       // 16-byte loads per thread in flight

__global__ __launch_bounds__(SCAN_THREADS) void k_overflow_scan(const uint16_t *__restrict__ cnt, int T, int nt,
                                                               int cap, uint8_t *__restrict__ row_flag,
                                                               int *__restrict__ ovf_rows, int ovf_cap,
                                                               int *__restrict__ n_ovf, bool tile_major) {
  __shared__ __align__(16) uint32_t flag4[SCAN_CHUNK / 4];
  __shared__ int wcount[SCAN_THREADS / 64];
  uint8_t *flag = reinterpret_cast<uint8_t *>(flag4);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int r0 = 0; r0 < T; r0 += SCAN_CHUNK) {
    const int nr = min(SCAN_CHUNK, T - r0);
    for (int i = tid; i < SCAN_CHUNK / 4; i += SCAN_THREADS) flag4[i] = 0u;
    __syncthreads();
    // counts of rows [r0, r0 + nr): row-major, the elements [r0 nt, (r0 + nr)
    // nt) of the flat array (one segment, element e of row e / nt);
    // tile-major, the elements [k T + r0, k T + r0 + nr) of each tile k (nt
    // segments, element e of row e - k T)
    const int nseg = tile_major ? nt : 1;
    for (int sg = 0; sg < nseg; ++sg) {
      const size_t e_begin = tile_major ? (size_t)sg * T + r0 : (size_t)r0 * nt;
      const size_t e_end = tile_major ? e_begin + nr : (size_t)(r0 + nr) * nt;
      const size_t row_base = tile_major ? e_begin : 0;
      const int rdiv = tile_major ? 1 : nt, rsub = tile_major ? 0 : r0;
      auto mark = [&](size_t e) { flag[(int)((e - row_base) / rdiv) - rsub] = 1; };
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(cnt + e_begin);
      const size_t head = min((size_t)(((16u - (a0 & 15u)) & 15u) / 2u), e_end - e_begin);
      const size_t v0 = e_begin + head;
      const size_t nv = (e_end - v0) / 8;  // whole 16-byte chunks
      const size_t v_end = v0 + nv * 8;
      for (size_t e = e_begin + tid; e < v0; e += SCAN_THREADS)
        if (cnt[e] > cap) mark(e);
      for (size_t e = v_end + tid; e < e_end; e += SCAN_THREADS)
        if (cnt[e] > cap) mark(e);
      for (size_t c0 = tid; c0 < nv; c0 += (size_t)SCAN_THREADS * SCAN_LOADS) {
        u32x4_t w[SCAN_LOADS];
#pragma unroll
        for (int q = 0; q < SCAN_LOADS; ++q) {
          const size_t c = c0 + (size_t)q * SCAN_THREADS;
          w[q] = c < nv ? *reinterpret_cast<const u32x4_t *>(cnt + v0 + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < SCAN_LOADS; ++q) {
          uint32_t mx = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = max(mx, max(w[q][j] & 0xFFFFu, w[q][j] >> 16));
          if (mx > (uint32_t)cap) {
            const size_t e0 = v0 + (c0 + (size_t)q * SCAN_THREADS) * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (((w[q][j / 2] >> (16 * (j & 1))) & 0xFFFFu) > (uint32_t)cap) mark(e0 + j);
          }
        }
      }
    }
    __syncthreads();
    // compaction: thread tid owns the flags of rows r0 + 8 tid .. r0 + 8 tid + 7
    const u32x2_t fw = reinterpret_cast<const u32x2_t *>(flag4)[tid];
    int c = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) c += ((fw[j / 4] >> (8 * (j % 4))) & 0xFFu) != 0;
    const int incl = wave_incl_scan(c);
    if (lane == 63) wcount[wave] = incl;
    __syncthreads();
    int pos = carry + incl - c, total = 0;
    for (int w = 0; w < SCAN_THREADS / 64; ++w) {
      pos += (w < wave) ? wcount[w] : 0;
      total += wcount[w];
    }
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) {
      const int rr = SCAN_PER * tid + j;
      if (rr < nr) {
        const bool f = ((fw[j / 4] >> (8 * (j % 4))) & 0xFFu) != 0;
        if (row_flag != nullptr) row_flag[r0 + rr] = f ? 1 : 0;
        if (f) {
          if (pos < ovf_cap) ovf_rows[pos] = r0 + rr;
          ++pos;
        }
      }
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_ovf = carry;
}

hipError_t overflow_scan(const ScanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_overflow_scan, dim3(1), dim3(SCAN_THREADS), 0, s, a.cnt, a.T, a.nt, a.cap, a.row_flag,
                     a.ovf_rows, a.ovf_cap, a.n_ovf, a.tile_major);
  return hipGetLastError();
}

// Ascending list of the rows whose flag is set; one workgroup, 8 consecutive
// flags per thread per round (thread order = row order).  Flags are bytes
// (written by the up kernel into the workspace) or int32 words.  With int32
// flags the list may overwrite the flag array itself: the list position of a
// row never exceeds the row's index, and every thread reads the round's flags
// before the barrier that precedes the round's writes.
constexpr int COMPACT_THREADS = 1024;
constexpr int COMPACT_PER = 8;

template <class FlagT>
__device__ __forceinline__ void load_flags(const FlagT *row_flag, int t0, int T, uint32_t (&f)[COMPACT_PER]);
template <>
__device__ __forceinline__ void load_flags<uint8_t>(const uint8_t *row_flag, int t0, int T,
                                                   uint32_t (&f)[COMPACT_PER]) {
  if (t0 + COMPACT_PER <= T && (reinterpret_cast<uintptr_t>(row_flag + t0) & 7) == 0) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(row_flag + t0);
#pragma unroll
    for (int q = 0; q < COMPACT_PER; ++q) f[q] = (w[q / 4] >> (8 * (q % 4))) & 0xFFu;
  } else {
#pragma unroll
    for (int q = 0; q < COMPACT_PER; ++q) f[q] = t0 + q < T ? row_flag[t0 + q] : 0u;
  }
}
template <>
__device__ __forceinline__ void load_flags<int>(const int *row_flag, int t0, int T, uint32_t (&f)[COMPACT_PER]) {
  if (t0 + COMPACT_PER <= T && (reinterpret_cast<uintptr_t>(row_flag + t0) & 15) == 0) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(row_flag + t0);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(row_flag + t0 + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[q] = a[q];
      f[q + 4] = b[q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < COMPACT_PER; ++q) f[q] = t0 + q < T ? (uint32_t)row_flag[t0 + q] : 0u;
  }
}

template <class FlagT>
__global__ __launch_bounds__(COMPACT_THREADS) void k_compact_rows(const FlagT *row_flag, int T, int *ovf_rows,
                                                                  int ovf_cap, int *__restrict__ n_ovf) {
  __shared__ int wcount[COMPACT_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < T; base += COMPACT_THREADS * COMPACT_PER) {
    const int t0 = base + tid * COMPACT_PER;
    uint32_t f[COMPACT_PER];
    load_flags<FlagT>(row_flag, t0, T, f);
    int c = 0;
#pragma unroll
    for (int q = 0; q < COMPACT_PER; ++q) c += f[q] != 0;
    const int incl = wave_incl_scan(c);
    if (lane == 63) wcount[wave] = incl;
    __syncthreads();
    int pos = carry + incl - c, total = 0;
    for (int w = 0; w < COMPACT_THREADS / 64; ++w) {
      pos += (w < wave) ? wcount[w] : 0;
      total += wcount[w];
    }
#pragma unroll
    for (int q = 0; q < COMPACT_PER; ++q) {
      if (f[q] != 0) {
        if (pos < ovf_cap) ovf_rows[pos] = t0 + q;
        ++pos;
      }
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_ovf = carry;
}

hipError_t compact_rows(const uint8_t *row_flag, int T, int *ovf_rows, int ovf_cap, int *n_ovf, hipStream_t s) {
  hipLaunchKernelGGL(k_compact_rows<uint8_t>, dim3(1), dim3(COMPACT_THREADS), 0, s, row_flag, T, ovf_rows, ovf_cap,
                     n_ovf);
  return hipGetLastError();
}

hipError_t compact_rows_in_place(int *flags_then_rows, int T, int *n_ovf, hipStream_t s) {
  hipLaunchKernelGGL(k_compact_rows<int>, dim3(1), dim3(COMPACT_THREADS), 0, s, flags_then_rows, T, flags_then_rows,
                     T, n_ovf);
  return hipGetLastError();
}

__global__ void k_zero_int(int *p) { *p = 0; }
__global__ void k_fill_f32(float *p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}
hipError_t zero_int(int *p, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_int, dim3(1), dim3(1), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sparse up projection.  DC = parts of d (1 or 2, UpPlan): the wave of
// (group, part q, token) dots the part's d / DC columns of x_t and of the
// W_u^T rows.  NC = 16-byte chunks per lane covering one part; U = entries in
// flight per wave (U * NC 16-byte loads per lane outstanding).
//
// Writes, per non-overflow row t, the compact entry list of the row, in
// ascending (tile, slot) order, i.e. ascending j:
//   DC = 1: list[t * stride + e] = (byte offset of hidden unit j's weight row,
//           v = round(h * u): fp32 bits, or bf16 bits in the low half);
//   DC = 2: list[t * stride + e] = (offset, u over the first half of d,
//           h, u over the second half): part 0 writes the first 8 bytes,
//           part 1 the last 8; the down kernel forms v = round(h * (u0 + u1));
// for e < list_n[t], and padding entries (NO_ROW, 0...) up to the next
// multiple of LIST_PAD.  With u_out non-null the wave also saves u of every entry at
// its TwELL slot: DC = 1 stores it, DC = 2 adds each half's partial sum to a
// slot zeroed beforehand (two fp32 addends: the sum does not depend on their
// order); the slots of an overflow row get NaN.  A row overflows
// iff one of its tiles counts more than cap entries; every wave decides that
// from the row's counts, skips such rows, and the group-0 wave records
// row_flag[t] (1 for an overflow row) and list_n[t] = -1 for them.  A local
// column index is taken modulo the tile width, so a malformed index cannot
// address a row outside its tile.  A (row, group) wave keeps the group's
// entries in LDS while it computes them and then writes them to the row's
// list with coalesced stores, 64 entries per instruction (the kernel is bound
// by its vector-memory instruction rate).

struct UpEntry {
  uint32_t off;   // byte offset of the unit's row in W_u^T (and in W_d)
  uint32_t dst;   // the entry's index in the compact list; once computed, the
                  // entry's second word (v, or its part's partial u)
  float h;        // the gate activation
  uint32_t slot;  // the entry's TwELL slot (where u is saved)
};

template <Dt D, int NC, int U, int DC>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_up(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wu,
    const uint16_t *__restrict__ cnt, const typename DtT<D>::T *__restrict__ val,
    const uint8_t *__restrict__ idx, uint8_t *__restrict__ row_flag, void *__restrict__ list_v,
    int *__restrict__ list_n, int stride, int T, int d, int nt, int tile, int cap, int tpg, int n_groups,
    int tok_per_wg, int n_tb, float *__restrict__ u_out) {
  using TT = typename DtT<D>::T;
  constexpr int EPC = 16 / sizeof(TT);  // elements per 16-byte chunk
  static_assert(DC == 1 || DC == 2, "d whole or in two halves");
  __shared__ UpEntry lists[SP_WAVES][UP_LIST];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int vg, tb;
  group_coords(blockIdx.x, n_groups * DC, n_tb, vg, tb);
  if (vg >= n_groups * DC) return;
  const int g = vg / DC, part = vg - g * DC;  // the two parts of a group sit on neighbouring XCDs
  const int k0 = g * tpg;
  const int kn = min(tpg, nt - k0);
  UpEntry *L = lists[wave];
  const int dp = d / DC;  // columns of one part
  u32x2_t *list = reinterpret_cast<u32x2_t *>(list_v);  // DC = 2: two u32x2 per entry
  // W_u^T from the part's first column on, to the end of the array
  const __amdgpu_buffer_rsrc_t wur =
      buffer_rsrc(wu + part * dp, ((size_t)nt * tile * d - (size_t)part * dp) * sizeof(TT));
  const uint32_t lane_off = lane * 16;
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);
  // lanes 16 r (r = 0..3) store the entry whose total their row holds
  const int my_u = Reduce<U>::entry(lane >> 4);
  const bool storer = (lane & 15) == 0 && (U == 4 || (lane & 31) == 0);

  for (int it = wave; it < tok_per_wg; it += SP_WAVES) {
    const int t = tb * tok_per_wg + it;
    if (t >= T) break;
    const TT *xt = x + (size_t)t * d + part * dp;
    u32x4_t xr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xr[c] = *reinterpret_cast<const u32x4_t *>(xt + (c * 64 + lane) * EPC);

    // Overflow test and entry counts from the row's tile counts: entries in
    // tiles before the group (where its entries start in the list), and for
    // group 0 the row total.
    const uint16_t *crow = cnt + (size_t)t * nt;
    const size_t lbase = (size_t)t * stride;
    const int k_end = g == 0 ? nt : k0;
    int partial = 0, c_first = 0;
    bool over = false;
    for (int kb = 0; kb < nt; kb += 64) {
      const int kk = kb + lane;
      const int c = kk < nt ? (int)crow[kk] : 0;
      if (kb == 0) c_first = c;
      over |= c > cap;
      partial += kk < k_end ? min(c, cap) : 0;
    }
    const bool ovf = ballot(over) != 0;
    const int sum = __builtin_amdgcn_readlane(wave_incl_scan(partial), 63);
    if (g == 0 && part == 0) {
      if (lane == 0) {
        row_flag[t] = ovf ? 1 : 0;
        list_n[t] = ovf ? -1 : sum;
      }
      if (!ovf && lane < ((sum + LIST_PAD - 1) & ~(LIST_PAD - 1)) - sum) {
        list[(lbase + sum + lane) * DC] = u32x2_t{NO_ROW, 0u};
        if constexpr (DC == 2) list[(lbase + sum + lane) * 2 + 1] = u32x2_t{0u, 0u};
      }
    }
    const size_t gslot0 = ((size_t)t * nt + k0) * cap;  // first slot of the group
    if (ovf) {
      if (u_out != nullptr && part == 0)
        for (int q = lane; q < kn * cap; q += 64) u_out[gslot0 + q] = __builtin_nanf("");
      continue;
    }
    const int before = g == 0 ? 0 : sum;
    // The group's entries into the wave list.  Tile k0 + q has n(q) entries
    // (lane q, q < kn <= 64); its slots are contiguous after those of tile q-1,
    // so the wave loads all kn * cap slots with one lane per slot and files
    // the occupied ones at (entries of the tiles before q) + slot.
    // the group's tile counts: from the registers of the pass above when the
    // row has at most 64 tiles
    const int cg = nt <= 64 ? __shfl(c_first, min(k0 + lane, 63), 64) : (lane < kn ? (int)crow[k0 + lane] : 0);
    const int n = lane < kn ? min(cg, cap) : 0;
    const int incl = wave_incl_scan(n);
    const int E = __builtin_amdgcn_readlane(incl, 63);
    for (int q0 = 0; q0 < kn * cap; q0 += 64) {
      const int q = q0 + lane;
      const int kq = q / cap, sq = q - kq * cap;
      const int nq = __shfl(n, kq & 63, 64);
      const int oq = __shfl(incl - n, kq & 63, 64) + sq;
      if (q < kn * cap && sq < nq) {
        UpEntry en;
        en.off = (uint32_t)((k0 + kq) * tile + (idx[gslot0 + q] & (tile - 1))) * row_bytes;
        en.dst = (uint32_t)(before + oq);
        en.h = to_f32(val[gslot0 + q]);
        en.slot = (uint32_t)(gslot0 + q);
        L[oq] = en;
      }
    }
    wave_sync_lds();

    for (int e0 = 0; e0 < E; e0 += 64) {
      const int ne = min(64, E - e0);
      const uint32_t moff = L[min(e0 + lane, E - 1)].off;
      for (int u0 = 0; u0 < ne; u0 += U) {
        u32x4_t w[U][NC];
        if (u0 + U <= ne) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint32_t off = read_lane(moff, u0 + u);
#pragma unroll
            for (int c = 0; c < NC; ++c) w[u][c] = buffer_load<u32x4_t>(wur, lane_off + c * 1024, off);
          }
        } else {  // last batch: no loads for its missing entries
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (u0 + u < ne) {
              const uint32_t off = read_lane(moff, u0 + u);
#pragma unroll
              for (int c = 0; c < NC; ++c) w[u][c] = buffer_load<u32x4_t>(wur, lane_off + c * 1024, off);
            } else {
#pragma unroll
              for (int c = 0; c < NC; ++c) w[u][c] = u32x4_t{0u, 0u, 0u, 0u};
            }
          }
        }
        const UpEntry mine = L[e0 + min(u0 + my_u, ne - 1)];
        float p[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u] = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) p[u] = dot16(xr[c], w[u][c], p[u], TT());
        }
        const float tot = Reduce<U>::run(p);
        if (storer && u0 + my_u < ne) {
          // the entry's second word goes to its dst field; the list is
          // written below, 64 entries per store
          if constexpr (DC == 1) {
            const float v = mine.h * tot;
            L[e0 + u0 + my_u].dst = D == Dt::BF16 ? (uint32_t)bf16_rne(v) : __float_as_uint(v);
            if (u_out != nullptr) u_out[mine.slot] = tot;
          } else {
            L[e0 + u0 + my_u].dst = __float_as_uint(tot);
            if (u_out != nullptr) atomicAdd(u_out + mine.slot, tot);
          }
        }
      }
    }
    wave_sync_lds();
    // the group's entries to the row's list: E consecutive entries from
    // position `before`
    for (int e = lane; e < E; e += 64) {
      const UpEntry en = L[e];
      if constexpr (DC == 1)
        list[lbase + before + e] = u32x2_t{en.off, en.dst};
      else
        list[(lbase + before + e) * 2 + part] = part == 0 ? u32x2_t{en.off, en.dst} : u32x2_t{__float_as_uint(en.h), en.dst};
    }
    wave_sync_lds();
  }
}

// ---------------------------------------------------------------------------
// Sparse down projection over the compact lists.  Every workgroup covers one
// SLICE-column slice of y; each lane loads 16 bytes of a W_d row per
// instruction (the vector memory pipeline's cost is per instruction, so wide
// loads matter), SLICE / (16 / s) lanes per entry: for bf16 and 256 columns
// the two half-waves take two different entries, for fp32 the whole wave
// takes one.  The token's list goes through LDS, 64 entries per load.
// U = load instructions in flight per wave.

template <Dt D, int SLICE, int U, int DC>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_down(
    const void *__restrict__ list_v, const int *__restrict__ list_n, int stride,
    const typename DtT<D>::T *__restrict__ wd, typename DtT<D>::T *__restrict__ y, int T, int d, int F,
    int n_slices, int tok_per_wg, int n_tb) {
  using TT = typename DtT<D>::T;
  constexpr int CPL = 16 / sizeof(TT);      // columns per lane
  constexpr int LPE = SLICE / CPL;          // lanes per entry
  constexpr int EPI = 64 / LPE;             // entries per load instruction
  constexpr int STEP = U * EPI;             // entries per iteration
  static_assert(EPI == 1 || EPI == 2, "32 or 64 lanes per entry");
  static_assert(D != Dt::BF16 || U % 2 == 0, "bf16 pairs the entries of one lane");
  static_assert(STEP <= 64 && 64 % STEP == 0, "a 64-entry chunk holds whole iterations");
  // One iteration consumes STEP list entries and a chunk holds the list's
  // entries rounded up to a multiple of LIST_PAD (the padding the up kernel
  // writes, whose loads return zeros); a larger STEP would read entries past
  // them and load weight rows at stale offsets.
  static_assert(LIST_PAD % STEP == 0, "STEP must divide the list padding");
  __shared__ u32x2_t chunk[SP_WAVES][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int part = lane / LPE;                 // which of the EPI entries this lane works on
  const int lcol = (lane % LPE) * CPL;         // lane's first column in the slice
  int sl, tb;
  group_coords(blockIdx.x, n_slices, n_tb, sl, tb);
  if (sl >= n_slices) return;
  // the slice's columns of row 0 onwards, to the end of W_d
  const __amdgpu_buffer_rsrc_t wdr =
      buffer_rsrc(wd + sl * SLICE, ((size_t)F * d - (size_t)sl * SLICE) * sizeof(TT));
  const uint32_t lane_off = lcol * sizeof(TT);
  u32x2_t *C = chunk[wave];
  for (int it = wave; it < tok_per_wg; it += SP_WAVES) {
    const int t = __builtin_amdgcn_readfirstlane(tb * tok_per_wg + it);
    if (t >= T) break;
    const int n = list_n[t];
    if (n < 0) continue;  // overflow row: the dense fallback writes it
    const u32x2_t *lt = reinterpret_cast<const u32x2_t *>(list_v) + (size_t)t * stride * DC;
    float acc[CPL];
#pragma unroll
    for (int v = 0; v < CPL; ++v) acc[v] = 0.f;
    for (int e0 = 0; e0 < n; e0 += 64) {
      // 64 entries of the list to LDS with one load; each lane then reads the
      // entry it works on (lanes of a half-wave read the same one), so the
      // row offset and the weight arrive per lane without any selects.  The
      // list is padded to a multiple of LIST_PAD entries with (NO_ROW, 0), whose
      // loads return zeros, so padding adds exactly 0 whatever the weights
      // hold; entries beyond that in the chunk are never read.
      const int ne = min(64, (n - e0 + LIST_PAD - 1) & ~(LIST_PAD - 1));
      if (lane < ne) {
        if constexpr (DC == 1) {
          C[lane] = lt[e0 + lane];
        } else {
          // (offset, u of the first half of d, h, u of the second half):
          // v = round(h * u), the halves added in a fixed order
          const u32x4_t q = reinterpret_cast<const u32x4_t *>(lt)[e0 + lane];
          const float v = __uint_as_float(q[2]) * (__uint_as_float(q[1]) + __uint_as_float(q[3]));
          C[lane] = u32x2_t{q[0], D == Dt::BF16 ? (uint32_t)bf16_rne(v) : __float_as_uint(v)};
        }
      }
      wave_sync_lds();
      for (int e = 0; e < ne; e += STEP) {
        u32x4_t w[U];
        uint32_t sw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const u32x2_t en = C[e + EPI * u + part];
          sw[u] = en[1];
          w[u] = buffer_load<u32x4_t>(wdr, lane_off + en[0], 0u);
        }
        if constexpr (D == Dt::BF16) {
          // entries 2p and 2p+1 of this lane: one dword holds their two v
          // (bf16), and per weight dword the same column of both rows is
          // paired, so one dot2 adds both products into that column
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
          for (int p = 0; p < U / 2; ++p) {
            const uint32_t vv = __builtin_amdgcn_perm(sw[2 * p + 1], sw[2 * p], 0x05040100u);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t wa = w[2 * p][q], wb = w[2 * p + 1][q];
              const uint32_t lo = __builtin_amdgcn_perm(wb, wa, 0x05040100u);  // column 2q of both rows
              const uint32_t hi = __builtin_amdgcn_perm(wb, wa, 0x07060302u);  // column 2q + 1
              acc[2 * q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo),
                                                          __builtin_bit_cast(bf16x2_t, vv), acc[2 * q], false);
              acc[2 * q + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi),
                                                              __builtin_bit_cast(bf16x2_t, vv), acc[2 * q + 1],
                                                              false);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = fmaf(__uint_as_float(sw[u]), __uint_as_float(w[u][v]), acc[v]);
          }
        }
      }
      wave_sync_lds();
    }
    // lanes l and l + 32 hold the same columns for the even and the odd
    // entries: add the halves
    if constexpr (EPI == 2) {
#pragma unroll
      for (int v = 0; v < CPL; ++v) {
        auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[v]), __float_as_uint(acc[v]), false, false);
        acc[v] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
      }
    }
    u32x4_t out;
    if constexpr (D == Dt::BF16) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        out[v] = (uint32_t)bf16_rne(acc[2 * v]) | ((uint32_t)bf16_rne(acc[2 * v + 1]) << 16);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) out[v] = __float_as_uint(acc[v]);
    }
    if (part == 0) *reinterpret_cast<u32x4_t *>(y + (size_t)t * d + sl * SLICE + lcol) = out;
  }
}

// ---------------------------------------------------------------------------
// Launchers.

template <Dt D, int NC, int DC>
static hipError_t launch_up(const SparseArgs &a, const UpPlan &p, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int nt = a.F / a.tile;
  const int tok = 16;
  const int n_tb = (a.T + tok - 1) / tok;
  constexpr int U = NC <= 4 ? 4 : 2;
  if (DC == 2 && a.u != nullptr) {  // the halves are added into zeroed slots
    const size_t n = (size_t)a.T * nt * a.cap;
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)std::min<size_t>((n + 255) / 256, 4096)), dim3(256), 0, s, a.u,
                       n, 0.0f);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_sparse_up<D, NC, U, DC>), dim3(padded_groups(p.n_groups * DC) * n_tb), dim3(SP_THREADS), 0,
                     s, (const TT *)a.x, (const TT *)a.wu, a.cnt, (const TT *)a.val, a.idx, a.row_flag, a.list,
                     a.list_n, a.stride, a.T, a.d, nt, a.tile, a.cap, p.tpg, p.n_groups, tok, n_tb, a.u);
  return hipGetLastError();
}

template <Dt D>
static hipError_t up_dispatch(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  // Tiles per group: about 4 MB of W_u^T rows per group (one XCD's L2); at
  // the 1.5B-class and larger layer shapes this was the fastest setting of a
  // sweep over 1..8 tiles per group.
  const UpPlan p = up_plan(a.d, a.F, a.tile, a.cap, a.dtype);
  const int nc = a.d / p.dc / (64 * (16 / (int)sizeof(TT)));
  if (p.dc == 2) {
    switch (nc) {
#define TWELL_UP2_CASE(N) \
  case N:                 \
    return launch_up<D, N, 2>(a, p, s);
      TWELL_UP2_CASE(1) TWELL_UP2_CASE(2) TWELL_UP2_CASE(3) TWELL_UP2_CASE(4) TWELL_UP2_CASE(5)
      TWELL_UP2_CASE(6) TWELL_UP2_CASE(7) TWELL_UP2_CASE(8)
#undef TWELL_UP2_CASE
      default:
        return hipErrorInvalidValue;
    }
  }
  switch (nc) {
#define TWELL_UP_CASE(N) \
  case N:                \
    return launch_up<D, N, 1>(a, p, s);
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

template <Dt D, int SLICE, int U, int DC>
static hipError_t launch_down(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int n_slices = a.d / SLICE;
  const int tok = 16;
  const int n_tb = (a.T + tok - 1) / tok;
  hipLaunchKernelGGL((k_sparse_down<D, SLICE, U, DC>), dim3(padded_groups(n_slices) * n_tb), dim3(SP_THREADS), 0, s,
                     a.list, a.list_n, a.stride, (const TT *)a.wd, (TT *)a.y, a.T, a.d, a.F, n_slices, tok, n_tb);
  return hipGetLastError();
}

hipError_t sparse_down(const SparseArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  // 256-column output slices, 8 list entries per iteration.  (128-column
  // slices, which would keep F rows of a slice within one XCD's L2 for
  // F > 8192, measured slower at F = 14336.)
  const int dc = up_plan(a.d, a.F, a.tile, a.cap, a.dtype).dc;
  if (a.dtype == Dt::BF16)
    return dc == 2 ? launch_down<Dt::BF16, 256, 8, 2>(a, s) : launch_down<Dt::BF16, 256, 8, 1>(a, s);
  return dc == 2 ? launch_down<Dt::F32, 256, 8, 2>(a, s) : launch_down<Dt::F32, 256, 8, 1>(a, s);
}

}  // namespace twell
