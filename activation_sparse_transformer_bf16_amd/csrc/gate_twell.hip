// Gate matmul with the TwELL epilogue.
//
// pre[t][j] = sum_k x[t][k] * w_gate[j][k] + beta[t] on the matrix cores; the
// epilogue rounds every value to the storage dtype, applies ReLU and writes
// the TwELL matrix of the tile straight from the accumulator registers.  This
// is the "sparsity materialised in the epilogue of the dense matmul, no
// separate conversion pass and no synchronisation between workgroups" design
// of gist.science "Sparser, Faster, Lighter Transformer Language Models",
// Resumen Técnico §2.A, carried over to gfx950: the N tile of the matmul is
// exactly one TwELL tile, so every (row, tile) pair is owned by one workgroup;
// the activity masks and the rounded tile are staged in the LDS the mainloop
// no longer needs, and one lane per 32-column mask word of a row compacts it
// in ascending column order.
#include "gemm.hpp"
#include "launch.hpp"

#include <algorithm>

namespace twell {

// LDS layout of the TwELL epilogue (RPP = rows per pass: 256, 128 or 64, the
// largest whose layout fits the 160 KB of LDS for the given cap):
//   masks  [256 rows][MW dwords]   activity bits of the whole tile (MW = BN/32)
//   tile   [BN cols][RS bytes]     rounded values of RPP rows, column-major
//   vals   [RPP][VS bytes]         slot values of each row of the pass
//   idxs   [RPP][IS bytes]         slot column offsets
//   dummy  [64][4 bytes]           where the lanes that hold no mask word write
template <Dt D, int BN, int RPP_, int BM = GEMM_BM>
struct EpilogueLds {
  using T = typename DtT<D>::T;
  static constexpr int S = (int)sizeof(T);
  static constexpr int MW = BN / 32;
  static constexpr int RPP = RPP_;
  static constexpr int RS = RPP * S + 8;
  static constexpr int MASKS = BM * MW * 4;
  static constexpr int TILE_OFF = MASKS;
  static constexpr int TILE = BN * RS;
  __host__ __device__ static constexpr int vs(int cap) { return (cap * S + 15) / 16 * 16; }
  __host__ __device__ static constexpr int is(int cap) { return (cap + 15) / 16 * 16; }
  __host__ __device__ static constexpr int vals_off() { return (TILE_OFF + TILE + 15) / 16 * 16; }
  __host__ __device__ static constexpr int idxs_off(int cap) { return vals_off() + RPP * vs(cap); }
  __host__ __device__ static constexpr int dummy_off(int cap) { return idxs_off(cap) + RPP * is(cap); }
  __host__ __device__ static constexpr int bytes(int cap) { return dummy_off(cap) + 64 * 4; }
};
constexpr int LDS_MAX = 160 * 1024;  // per CU; a DmaHalf workgroup gets half of it

// Four consecutive rows (accumulator registers i0..i0+3) of one column, rounded.
__device__ __forceinline__ void put4(char *dst, const f32x16_t &a, int i0, uint16_t) {
  const uint32_t lo = (uint32_t)bf16_rne(a[i0]) | ((uint32_t)bf16_rne(a[i0 + 1]) << 16);
  const uint32_t hi = (uint32_t)bf16_rne(a[i0 + 2]) | ((uint32_t)bf16_rne(a[i0 + 3]) << 16);
  *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{lo, hi};
}
__device__ __forceinline__ void put4(char *dst, const f32x16_t &a, int i0, float) {
  *reinterpret_cast<f32x2_t *>(dst) = f32x2_t{a[i0], a[i0 + 1]};
  *reinterpret_cast<f32x2_t *>(dst + 8) = f32x2_t{a[i0 + 2], a[i0 + 3]};
}

// v shifted by a DPP row shift (CTRL), or 0 where `take` is false.  The DPP
// move runs with every lane active (a lane can only read an active lane), the
// selection after it.
template <int CTRL>
__device__ __forceinline__ int seg_shift_add(int v, bool take) {
  int sh = __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
  asm volatile("" : "+v"(sh));
  return take ? sh : 0;
}

// LDS writes of a wave visible to the whole wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copy one chunk of `unit` (16, 4, 2 or 1) bytes LDS -> global.
__device__ __forceinline__ void copy_chunk(char *__restrict__ g, const char *l, int unit) {
  if (unit == 16)
    *reinterpret_cast<u32x4_t *>(g) = *reinterpret_cast<const u32x4_t *>(l);
  else if (unit == 4)
    *reinterpret_cast<uint32_t *>(g) = *reinterpret_cast<const uint32_t *>(l);
  else if (unit == 2)
    *reinterpret_cast<uint16_t *>(g) = *reinterpret_cast<const uint16_t *>(l);
  else
    *g = *l;
}

template <Dt D, int BN, int RPP_, bool DUMP, class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::WAVES_PER_SIMD) void k_gate_twell(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wg,
    const float *__restrict__ beta, int M, int K, int N, int cap, uint16_t *__restrict__ cnt,
    typename DtT<D>::T *__restrict__ val, uint8_t *__restrict__ idx,
    typename DtT<D>::T *__restrict__ pre_out, bool tile_major) {
  using T = typename DtT<D>::T;
  using WT = WaveTile<BN, Cfg>;
  constexpr int NWM = WT::NWM, NWN = WT::NWN;
  constexpr int BM = Cfg::BM;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int mt = (M + BM - 1) / BM, ntl = N / BN;
  int tm, tn;
  tile_coords(blockIdx.x, mt, ntl, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = WT::row0(wave), col0 = WT::col0(wave);
  const size_t ldk = (size_t)K * sizeof(T);

  auto rowA = [&](int r) {
    const int row = min(m0 + r, M - 1);
    return reinterpret_cast<const char *>(x) + (size_t)row * ldk;
  };
  auto rowB = [&](int r) { return reinterpret_cast<const char *>(wg) + (size_t)(n0 + r) * ldk; };

  // The accumulators start at beta so that the matmul adds the gate bias.
  auto rowv = [&](int r) -> const float * { return beta != nullptr ? beta + min(m0 + r, M - 1) : nullptr; };
  auto init = [&](f32x16_t (&a)[NWM][NWN], const float *vals) {
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm) {
      f32x16_t b0;
#pragma unroll
      for (int i = 0; i < 16; ++i) b0[i] = vals != nullptr ? vals[acc_row(row0, bm, i, lane)] : 0.0f;
#pragma unroll
      for (int bn = 0; bn < NWN; ++bn) a[bm][bn] = b0;
    }
  };
  f32x16_t acc[NWM][NWN];
  gemm_mainloop_dma<D, BN, Cfg>(acc, rowA, rowB, rowv, init, (int)(ldk / SLAB), smem);

  // ---- TwELL epilogue ----
  // M  every wave compares its accumulators with the activity threshold of the
  //    rounded value (v_cmp, one 64-bit mask per register: 32 columns of two
  //    rows) and files the masks in LDS as BN-bit row masks;
  // then per pass of RPP rows (one pass when all 256 rows fit):
  //  V  the waves that own those rows stage the rounded values in LDS;
  //  C  MW lanes per row, one per 32-column mask word: a segmented prefix
  //     count over the row's words gives each word's first slot, each lane
  //     walks its word's set bits in ascending order (ffbl) and puts the
  //     (value, column) pairs that fall below `cap` in the row's LDS slots;
  //     then the row's count, slots and zero padding go to global memory
  //     with vector stores.
  using L = EpilogueLds<D, BN, RPP_, BM>;
  constexpr int MW = L::MW, RPP = L::RPP, RS = L::RS, S = L::S;
  const int ntiles = N / BN;
  const int VS = L::vs(cap), IS = L::is(cap);
  char *tile = smem + L::TILE_OFF;
  char *vals = smem + L::vals_off();
  char *idxs = smem + L::idxs_off(cap);
  uint32_t *masks = reinterpret_cast<uint32_t *>(smem);
  const int vunit = (cap * S) % 16 == 0 ? 16 : ((cap * S) % 4 == 0 ? 4 : S);
  const int iunit = cap % 16 == 0 ? 16 : (cap % 4 == 0 ? 4 : 1);
  // lane k < 2*NWN receives mask word col0/32 + k % NWN of row R (k < NWN)
  // or of row R+4
  const bool holder = lane < 2 * NWN;
  const int word = col0 / 32 + lane % NWN;
  const int roff = lane < NWN ? 0 : 4;
  uint32_t *dummy = reinterpret_cast<uint32_t *>(smem + L::dummy_off(cap)) + (tid & 63);
  auto put_masks = [&](int bm, int i) {
    uint32_t w = 0;
#pragma unroll
    for (int bn = 0; bn < NWN; ++bn) {
      const uint64_t m = ballot(active_after_round<D>(acc[bm][bn][i]));
      w = (lane == bn) ? (uint32_t)m : w;
      w = (lane == NWN + bn) ? (uint32_t)(m >> 32) : w;
    }
    const int R = row0 + 32 * bm + 8 * (i >> 2) + (i & 3);
    uint32_t *dst = holder ? masks + (R + roff) * MW + word : dummy;
    *dst = w;
  };
  // rounded values of rows 32 bm + 8 g + {0..3} (+4 for the upper half-wave)
  // of the wave's blocks, into the column-major tile of pass p
  auto put_values = [&](int p, int bm, int g) {
    const int rl0 = row0 - p * RPP + 4 * (lane >> 5);  // lane's first row, relative to the pass
#pragma unroll
    for (int bn = 0; bn < NWN; ++bn) {
      char *colp = tile + (col0 + 32 * bn + (lane & 31)) * RS;
      put4(colp + (rl0 + 32 * bm + 8 * g) * S, acc[bm][bn], 4 * g, T());
      if constexpr (DUMP) {
        const int t0 = m0 + p * RPP + rl0 + 32 * bm + 8 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (t0 + q < M)
            pre_out[(size_t)(t0 + q) * N + n0 + col0 + 32 * bn + (lane & 31)] = from_f32<D>(acc[bm][bn][4 * g + q]);
      }
    }
  };
  auto clear_slots = [&]() {
    for (int o = tid * 16; o < RPP * (VS + IS); o += Cfg::THREADS * 16)
      *reinterpret_cast<u32x4_t *>(vals + o) = u32x4_t{0u, 0u, 0u, 0u};
  };
  if constexpr (RPP == BM) {
    // one pass: masks and values from the same register reads
    clear_slots();
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        put_values(0, bm, g);
#pragma unroll
        for (int q = 0; q < 4; ++q) put_masks(bm, 4 * g + q);
      }
  } else {
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
      for (int i = 0; i < 16; ++i) put_masks(bm, i);
    // The accumulators are read again by V: make them opaque here so that
    // the copies made for the masks are not kept live (which would spill).
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
      for (int bn = 0; bn < NWN; ++bn) asm volatile("" : "+a"(acc[bm][bn]));
  }
#pragma unroll
  for (int p = 0; p < BM / RPP; ++p) {
    if constexpr (RPP != BM) {
      // V: stage the rounded values of this pass and clear the slots
      clear_slots();
#pragma unroll
      for (int bm = 0; bm < NWM; ++bm) {
        if ((row0 + 32 * bm) / RPP != p) continue;  // wave-uniform
#pragma unroll
        for (int g = 0; g < 4; ++g) put_values(p, bm, g);
      }
    }
    __syncthreads();
    // C: MW lanes per row (wsub = mask word), RPS rows per wave step
    constexpr int RPS = 64 / MW;
    static_assert(MW == 4 || MW == 8, "tile of 128 or 256 columns");
    const int wsub = lane % MW;
    const int nvc = (cap * S) / vunit, nic = cap / iunit;  // chunks of the slot values / indices
    for (int rl = wave * RPS + lane / MW; rl - lane / MW < RPP; rl += Cfg::WAVES * RPS) {
      const int rg = p * RPP + rl;  // row within the tile
      const int t = m0 + rg;
      uint32_t m = masks[rg * MW + wsub];
      const int c = __popc(m);
      // inclusive prefix count over the row's MW lanes (DPP row shifts; a
      // row of 16 lanes holds 16 / MW segments, lanes below the shift in a
      // segment add nothing); the last lane of the segment holds the total
      int incl = c;
      incl += seg_shift_add<0x111>(incl, wsub >= 1);    // row_shr 1
      incl += seg_shift_add<0x112>(incl, wsub >= 2);    // row_shr 2
      if constexpr (MW == 8) incl += seg_shift_add<0x114>(incl, wsub >= 4);  // row_shr 4
      int n = incl - c;
      while (m != 0 && n < cap) {
        const int col = 32 * wsub + __builtin_ctz(m);
        m &= m - 1;
        *reinterpret_cast<T *>(vals + rl * VS + n * S) = *reinterpret_cast<const T *>(tile + col * RS + rl * S);
        idxs[rl * IS + n] = (char)col;
        ++n;
      }
      wave_lds_sync();
      if (t < M) {
        // the (row, tile) record: row-major, or tile-major (the tile's rows contiguous)
        const size_t rec = tile_major ? (size_t)tn * M + t : (size_t)t * ntiles + tn;
        const size_t slot0 = rec * cap;
        if (wsub == MW - 1) cnt[rec] = (uint16_t)incl;
        for (int q = wsub; q < nvc + nic; q += MW) {
          if (q < nvc)
            copy_chunk(reinterpret_cast<char *>(val + slot0) + q * vunit, vals + rl * VS + q * vunit, vunit);
          else
            copy_chunk(reinterpret_cast<char *>(idx + slot0) + (q - nvc) * iunit, idxs + rl * IS + (q - nvc) * iunit,
                       iunit);
        }
      }
    }
    if (p + 1 < BM / RPP) __syncthreads();
  }
}

template <Dt D, int BN, int RPP, bool DUMP, class Cfg>
static hipError_t launch_gate(const GateArgs &a, hipStream_t s) {
  using T = typename DtT<D>::T;
  auto kern = k_gate_twell<D, BN, RPP, DUMP, Cfg>;
  const int lds = std::max(gemm_dma_lds_bytes<Cfg>(BN), EpilogueLds<D, BN, RPP, Cfg::BM>::bytes(a.cap));
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int mt = (a.M + Cfg::BM - 1) / Cfg::BM, ntl = a.N / BN;
  hipLaunchKernelGGL(kern, dim3(mt * ntl), dim3(Cfg::THREADS), lds, s, (const T *)a.x,
                     (const T *)a.wg, a.beta, a.M, a.K, a.N, a.cap, a.cnt, (T *)a.val, a.idx,
                     (T *)a.pre_out, a.tile_major);
  return hipGetLastError();
}

// The largest rows-per-pass whose epilogue layout fits the workgroup's share
// of the LDS for this cap (all of it for DmaBig, half for DmaHalf, which runs
// two workgroups per CU).
template <Dt D, int BN, bool DUMP, class Cfg>
static hipError_t launch_gate_rpp(const GateArgs &a, hipStream_t s) {
  constexpr int BM = Cfg::BM;
  constexpr int budget = BM == 256 ? LDS_MAX : LDS_MAX / 2;
  if (EpilogueLds<D, BN, BM, BM>::bytes(a.cap) <= budget) return launch_gate<D, BN, BM, DUMP, Cfg>(a, s);
  if (EpilogueLds<D, BN, 128, BM>::bytes(a.cap) <= budget) return launch_gate<D, BN, 128, DUMP, Cfg>(a, s);
  return launch_gate<D, BN, 64, DUMP, Cfg>(a, s);
}

template <Dt D, int BN, class Cfg>
static hipError_t launch_gate(const GateArgs &a, hipStream_t s) {
  return a.pre_out != nullptr ? launch_gate_rpp<D, BN, true, Cfg>(a, s) : launch_gate_rpp<D, BN, false, Cfg>(a, s);
}

hipError_t gate_twell(const GateArgs &a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.dtype == Dt::BF16) {
    if (a.tile == 256) return launch_gate<Dt::BF16, 256, DmaBig>(a, s);
    if (a.tile == 128) return launch_gate<Dt::BF16, 128, DmaBig>(a, s);
  } else {
    if (a.tile == 256) return launch_gate<Dt::F32, 256, DmaBig>(a, s);
    if (a.tile == 128) return launch_gate<Dt::F32, 128, DmaBig>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace twell
