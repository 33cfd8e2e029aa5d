// Standalone TwELL packing of an explicit pre-activation matrix, and the copy
// of the overflowing rows into the dense backup matrix.
//
// Format: gist.science "Sparser, Faster, Lighter Transformer Language Models",
// Resumen Técnico §2.A (column tiles, per-tile non-zeros; rows that overflow
// go to a dense backup matrix).  One wave packs one row.  Every lane loads 16
// bytes of the row per load instruction, so one load covers 64 * 16 bytes:
// one tile (fp32, 256 columns), two or four.  The lanes of a tile form a
// segment.  Per-element activity ballots counted over the lanes below (mbcnt),
// less the non-zeros of the earlier segments, give the ascending rank of each
// non-zero inside its tile.  The first `cap`
// non-zeros of a tile, their local columns and the tile's count are filed in
// a per-wave LDS image of the chunk's TwELL output (zero-initialised, so the
// padding is +0 / 0), which the wave then writes out with 16-byte stores.
// The pass streams the matrix once from HBM.  With a flag array, the wave also
// records whether its row overflows (some tile counts more than cap).
#include "gather.hpp"
#include "launch.hpp"

namespace twell {

constexpr int PACK_THREADS = 256;
constexpr int PACK_WAVES = PACK_THREADS / 64;
constexpr int PACK_LOADS = 8;  // 16-byte loads per lane in flight per chunk

__host__ __device__ constexpr int pack_align16(int n) { return (n + 15) & ~15; }

// Tiles per chunk (PACK_LOADS loads of 64 x 16 bytes) and the per-wave LDS
// bytes of one chunk's output image: values | local columns | counts.
__host__ __device__ constexpr int pack_chunk_tiles(int tile, int elem_bytes) {
  return PACK_LOADS * (64 / (tile / (16 / elem_bytes)));
}
__host__ __device__ constexpr int pack_stage_bytes(int tile, int elem_bytes, int cap) {
  return pack_align16(pack_chunk_tiles(tile, elem_bytes) * cap * elem_bytes) +
         pack_align16(pack_chunk_tiles(tile, elem_bytes) * cap) + pack_align16(pack_chunk_tiles(tile, elem_bytes) * 2);
}

// Wave-cooperative copy of n bytes from LDS to global memory, with the widest
// stores the destination's alignment and the length allow.
__device__ __forceinline__ void pack_copy_out(char *dst, const char *src, int n, int lane) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if ((a & 15) == 0 && (n & 15) == 0) {
    for (int o = lane * 16; o < n; o += 64 * 16)
      *reinterpret_cast<u32x4_t *>(dst + o) = *reinterpret_cast<const u32x4_t *>(src + o);
  } else if ((a & 3) == 0 && (n & 3) == 0) {
    for (int o = lane * 4; o < n; o += 64 * 4)
      *reinterpret_cast<uint32_t *>(dst + o) = *reinterpret_cast<const uint32_t *>(src + o);
  } else if ((a & 1) == 0 && (n & 1) == 0) {
    for (int o = lane * 2; o < n; o += 64 * 2)
      *reinterpret_cast<uint16_t *>(dst + o) = *reinterpret_cast<const uint16_t *>(src + o);
  } else {
    for (int o = lane; o < n; o += 64) dst[o] = src[o];
  }
}

template <class TT, int EPL>
__device__ __forceinline__ void unpack16(const u32x4_t &w, TT (&o)[EPL]) {
  if constexpr (sizeof(TT) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      o[2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(w[e]);
  }
}

template <Dt D, int TILE>
__global__ __launch_bounds__(PACK_THREADS) void k_pack(const typename DtT<D>::T *__restrict__ pre, int T, int F,
                                                      int cap, uint16_t *__restrict__ cnt,
                                                      typename DtT<D>::T *__restrict__ val,
                                                      uint8_t *__restrict__ idx, int *__restrict__ row_flag) {
  using TT = typename DtT<D>::T;
  constexpr int EPL = 16 / sizeof(TT);  // elements per lane per load
  constexpr int LPT = TILE / EPL;       // lanes per tile
  constexpr int TPL = 64 / LPT;         // tiles per load
  constexpr int CH = PACK_LOADS * TPL;  // tiles per chunk
  static_assert(CH == pack_chunk_tiles(TILE, sizeof(TT)), "chunk layout");
  extern __shared__ __align__(16) char pack_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * PACK_WAVES + wave;
  if (t >= T) return;
  const int nt = F / TILE;
  const int vbytes = pack_align16(CH * cap * (int)sizeof(TT)), ibytes = pack_align16(CH * cap);
  char *stage = pack_lds + wave * pack_stage_bytes(TILE, sizeof(TT), cap);
  TT *sv = reinterpret_cast<TT *>(stage);
  uint8_t *si = reinterpret_cast<uint8_t *>(stage + vbytes);
  uint16_t *sc = reinterpret_cast<uint16_t *>(stage + vbytes + ibytes);
  const int seg = lane / LPT, seg_lo = seg * LPT;
  // The row as a buffer of F * s bytes: loads past its last tile return 0 (the
  // range check covers the per-lane offset, which carries the whole offset).
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<TT *>(pre + (size_t)t * F), 0, F * (int)sizeof(TT), 0x00020000);
  const uint32_t voff = (uint32_t)(seg * TILE + (lane - seg_lo) * EPL) * sizeof(TT);
  bool ovf = false;
  for (int k0 = 0; k0 < nt; k0 += CH) {
    const int nch = min(CH, nt - k0);
    for (int o = lane * 16; o < vbytes + ibytes; o += 64 * 16)
      *reinterpret_cast<u32x4_t *>(stage + o) = u32x4_t{0u, 0u, 0u, 0u};
    u32x4_t raw[PACK_LOADS];
#pragma unroll
    for (int q = 0; q < PACK_LOADS; ++q)
      raw[q] = buffer_load<u32x4_t>(rsrc, voff + (uint32_t)((k0 + q * TPL) * TILE * sizeof(TT)), 0u);
    wave_sync_lds();
#pragma unroll
    for (int q = 0; q < PACK_LOADS; ++q) {
      const int kc = q * TPL + seg;  // tile inside the chunk
      TT v[EPL];
      unpack16<TT, EPL>(raw[q], v);
      bool act[EPL];
      uint32_t below = 0;  // non-zeros of this load in the lanes below (whole wave)
      int own = 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        act[e] = active_bits(v[e]);  // +0 for the lanes past the last tile: inactive
        const uint64_t m = ballot(act[e]);
        below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, below));
        own += act[e] ? 1 : 0;
      }
      // Non-zeros of the earlier segments (base) and up to the end of this
      // segment, read from the segments' first and last lanes.
      const int incl = (int)below + own;
      int base = 0, end = 0;
#pragma unroll
      for (int sg = 0; sg < TPL; ++sg) {
        const int b = sg == 0 ? 0 : __builtin_amdgcn_readlane((int)below, sg * LPT);
        const int en = __builtin_amdgcn_readlane(incl, sg * LPT + LPT - 1);
        if (seg == sg) {
          base = b;
          end = en;
        }
      }
      if (own > 0) {
        int r = (int)below - base;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          if (act[e]) {
            if (r < cap) {
              sv[kc * cap + r] = v[e];
              si[kc * cap + r] = (uint8_t)((lane - seg_lo) * EPL + e);
            }
            ++r;
          }
        }
      }
      if (lane == seg_lo) sc[kc] = (uint16_t)(end - base);
      ovf |= ballot(lane == seg_lo && end - base > cap) != 0;
    }
    wave_sync_lds();
    const size_t slot0 = ((size_t)t * nt + k0) * cap;
    pack_copy_out(reinterpret_cast<char *>(val + slot0), stage, nch * cap * (int)sizeof(TT), lane);
    pack_copy_out(reinterpret_cast<char *>(idx + slot0), reinterpret_cast<const char *>(si), nch * cap, lane);
    pack_copy_out(reinterpret_cast<char *>(cnt + (size_t)t * nt + k0), reinterpret_cast<const char *>(sc), nch * 2,
                  lane);
    wave_sync_lds();
  }
  if (row_flag != nullptr && lane == 0) row_flag[t] = ovf ? 1 : 0;
}

template <Dt D, int TILE>
static hipError_t launch_pack(const PackArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int blocks = (a.T + PACK_WAVES - 1) / PACK_WAVES;
  const int lds = PACK_WAVES * pack_stage_bytes(TILE, sizeof(TT), a.cap);
  hipLaunchKernelGGL((k_pack<D, TILE>), dim3(blocks), dim3(PACK_THREADS), lds, s, (const TT *)a.pre, a.T, a.F,
                     a.cap, a.cnt, (TT *)a.val, a.idx, a.row_flag);
  return hipGetLastError();
}

hipError_t pack_tiles(const PackArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.dtype == Dt::BF16) {
    if (a.tile == 256) return launch_pack<Dt::BF16, 256>(a, s);
    if (a.tile == 128) return launch_pack<Dt::BF16, 128>(a, s);
  } else {
    if (a.tile == 256) return launch_pack<Dt::F32, 256>(a, s);
    if (a.tile == 128) return launch_pack<Dt::F32, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// dense[r][:] = ReLU(pre[ovf_rows[r]][:]) for r < min(*n_ovf, ovf_cap), 16
// bytes per lane (rows are F * s bytes, a multiple of 256; both matrices are
// 16-byte aligned).  One workgroup per row at a time.
template <class TT>
__device__ __forceinline__ uint32_t relu_word(uint32_t w);
template <>
__device__ __forceinline__ uint32_t relu_word<uint16_t>(uint32_t w) {
  const uint32_t lo = active_bits((uint16_t)(w & 0xFFFFu)) ? (w & 0xFFFFu) : 0u;
  const uint32_t hi = active_bits((uint16_t)(w >> 16)) ? (w & 0xFFFF0000u) : 0u;
  return lo | hi;
}
template <>
__device__ __forceinline__ uint32_t relu_word<float>(uint32_t w) {
  return active_bits(__uint_as_float(w)) ? w : 0u;
}

constexpr int DENSE_ROWS_WGS = 512;

template <Dt D>
__global__ __launch_bounds__(256) void k_dense_rows(const typename DtT<D>::T *__restrict__ pre, int F,
                                                   const int *__restrict__ ovf_rows, const int *__restrict__ n_ovf,
                                                   int ovf_cap, typename DtT<D>::T *__restrict__ dense) {
  using TT = typename DtT<D>::T;
  const int n = min(*n_ovf, ovf_cap);
  const int chunks = F * (int)sizeof(TT) / 16;
  for (int r = blockIdx.x; r < n; r += gridDim.x) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(pre + (size_t)ovf_rows[r] * F);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(dense + (size_t)r * F);
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      const u32x4_t v = src[c];
      dst[c] = u32x4_t{relu_word<TT>(v[0]), relu_word<TT>(v[1]), relu_word<TT>(v[2]), relu_word<TT>(v[3])};
    }
  }
}

hipError_t pack_dense_rows(const DenseRowsArgs &a, hipStream_t s) {
  if (a.dense == nullptr || a.ovf_cap <= 0 || a.T <= 0) return hipSuccess;
  const int blocks = std::min(std::min(a.ovf_cap, a.T), DENSE_ROWS_WGS);
  if (a.dtype == Dt::BF16)
    hipLaunchKernelGGL(k_dense_rows<Dt::BF16>, dim3(blocks), dim3(256), 0, s, (const uint16_t *)a.pre, a.F,
                       a.ovf_rows, a.n_ovf, a.ovf_cap, (uint16_t *)a.dense);
  else
    hipLaunchKernelGGL(k_dense_rows<Dt::F32>, dim3(blocks), dim3(256), 0, s, (const float *)a.pre, a.F,
                       a.ovf_rows, a.n_ovf, a.ovf_cap, (float *)a.dense);
  return hipGetLastError();
}

}  // namespace twell
