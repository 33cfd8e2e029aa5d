// Standalone TwELL packing of an explicit pre-activation matrix, and the copy
// of the overflowing rows into the dense backup matrix.
//
// Format: gist.science "Sparser, Faster, Lighter Transformer Language Models",
// Resumen Técnico §2.A (column tiles, per-tile non-zeros; rows that overflow
// go to a dense backup matrix).  One wave packs one row, a chunk of
// PACK_LOADS loads at a time.  Every lane loads 16 bytes of the row per load
// instruction, so one load covers 64 * 16 bytes: one tile (fp32, 256
// columns), two or four.  The lanes of a tile form a segment.  Per load, each
// lane turns its elements into activity bits; a wave prefix sum of the lanes'
// counts, less the non-zeros of the earlier segments, gives the rank of the
// lane's first non-zero in its tile, and the segment ends give the tile
// counts.  After the chunk's loads, each lane walks its own non-zeros (few at
// high sparsity) in ascending column order and files the first `cap` of each
// tile, with their local columns, in a per-wave LDS image of the chunk's TwELL
// output (zero-initialised, so the padding is +0 / 0), which the wave then
// writes out with 16-byte stores.  The pass streams the matrix once from HBM.
// With a flag array, the wave also records whether its row overflows (some
// tile counts more than cap).
#include "gather.hpp"
#include "launch.hpp"

namespace twell {

constexpr int PACK_THREADS = 256;
constexpr int PACK_WAVES = PACK_THREADS / 64;
constexpr int PACK_LOADS = 8;  // 16-byte loads per lane in flight per chunk

__host__ __device__ constexpr int pack_align16(int n) { return (n + 15) & ~15; }

// Tiles per chunk (PACK_LOADS loads of 64 x 16 bytes) and the per-wave LDS
// bytes of one chunk: its output image (values | local columns | counts) and
// the stash of the loads of lanes that hold a non-zero ([PACK_LOADS][64][16]).
__host__ __device__ constexpr int pack_chunk_tiles(int tile, int elem_bytes) {
  return PACK_LOADS * (64 / (tile / (16 / elem_bytes)));
}
__host__ __device__ constexpr int pack_stage_bytes(int tile, int elem_bytes, int cap) {
  return pack_align16(pack_chunk_tiles(tile, elem_bytes) * cap * elem_bytes) +
         pack_align16(pack_chunk_tiles(tile, elem_bytes) * cap) + pack_align16(pack_chunk_tiles(tile, elem_bytes) * 2) +
         PACK_LOADS * 64 * 16;
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

// Activity of the EPL elements of a 16-byte load as bits, element 0 in the
// highest of the EPL bits (each step doubles and adds one flag).
template <class TT, int EPL>
__device__ __forceinline__ uint32_t active_mask16(const u32x4_t &w);
template <>
__device__ __forceinline__ uint32_t active_mask16<uint16_t, 8>(const u32x4_t &w) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bf16 bits b active iff 1 <= b <= 0x7F80, i.e. (b - 1) mod 2^16 < 0x7F80.
    // The element goes through a scalar: bit-casting a vector element
    // expression directly reads the vector's first element with this compiler.
    const uint32_t wk = w[k];
    const us2 m = __builtin_bit_cast(us2, wk) - (us2){1, 1};
    bits = bits + bits + (m.x < 0x7F80 ? 1u : 0u);
    bits = bits + bits + (m.y < 0x7F80 ? 1u : 0u);
  }
  return bits;
}
template <>
__device__ __forceinline__ uint32_t active_mask16<float, 4>(const u32x4_t &w) {
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) bits = bits + bits + (active_bits(__uint_as_float(w[k])) ? 1u : 0u);
  return bits;
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
  static_assert(PACK_LOADS * EPL <= 64 && PACK_LOADS <= 8, "a chunk's flags in 64 bits, its rank bases in 8 bytes");
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
  char *stash = stage + vbytes + ibytes + pack_align16(CH * 2);  // [PACK_LOADS][64 lanes][16 bytes]
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
    // Per load: the lane's active elements as bits, its rank base in the
    // tile (kept for the walk below, one byte per load), the tile counts;
    // lanes with an active element stash their 16 bytes for the walk.
    uint64_t all = 0;           // load q's bits at [(PACK_LOADS-1-q) * EPL, +EPL), element 0 highest
    uint32_t r0lo = 0, r0hi = 0;  // rank base of loads 0-3 and 4-7, a byte each
#pragma unroll
    for (int q = 0; q < PACK_LOADS; ++q) {
      const int kc = q * TPL + seg;  // tile inside the chunk
      uint32_t bits = active_mask16<TT, EPL>(raw[q]);  // +0 past the last tile: inactive
      const int own = __builtin_popcount(bits);
      const int incl = wave_incl_scan(own);
      // Non-zeros of the earlier segments (base) and up to the end of this
      // segment, read from the segments' last lanes.
      int base = 0, end = 0;
#pragma unroll
      for (int sg = 0; sg < TPL; ++sg) {
        const int b = sg == 0 ? 0 : __builtin_amdgcn_readlane(incl, sg * LPT - 1);
        const int en = __builtin_amdgcn_readlane(incl, sg * LPT + LPT - 1);
        if (seg == sg) {
          base = b;
          end = en;
        }
      }
      const int r0 = incl - own - base;  // rank of the lane's first non-zero in the tile
      if (r0 >= cap) bits = 0;            // past the tile's capacity: nothing to file
      if (bits != 0) *reinterpret_cast<u32x4_t *>(stash + (q * 64 + lane) * 16) = raw[q];
      all |= (uint64_t)bits << ((PACK_LOADS - 1 - q) * EPL);
      const uint32_t rb = bits != 0 ? (uint32_t)r0 : 0u;  // < cap <= 64 where it is read back
      if (q < 4)
        r0lo |= rb << (q * 8);
      else
        r0hi |= rb << ((q - 4) * 8);
      if (lane == seg_lo) sc[kc] = (uint16_t)(end - base);
      ovf |= ballot(lane == seg_lo && end - base > cap) != 0;
    }
    // The lane's non-zeros of the chunk in ascending (load, element) order,
    // i.e. ascending column inside each tile; k counts those of the same load
    // already filed.
    int cur = -1, k = 0;
    while (all != 0) {
      const int hb = 63 - __builtin_clzll(all);
      all ^= 1ull << hb;
      const int pos = PACK_LOADS * EPL - 1 - hb;
      const int q = pos / EPL, e = pos % EPL;
      k = q == cur ? k + 1 : 0;
      cur = q;
      const int r = (int)(((q < 4 ? r0lo : r0hi) >> ((q & 3) * 8)) & 0xFFu) + k;
      if (r < cap) {
        const int kc = q * TPL + seg;
        sv[kc * cap + r] = *reinterpret_cast<const TT *>(stash + (q * 64 + lane) * 16 + e * (int)sizeof(TT));
        si[kc * cap + r] = (uint8_t)((lane - seg_lo) * EPL + e);
      }
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
