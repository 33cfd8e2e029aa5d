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
// no longer needs, and one lane per row compacts it in ascending column order.
#include "gemm.hpp"
#include "launch.hpp"

#include <algorithm>

namespace twell {

// LDS layout of the TwELL epilogue:
//   masks  [256 rows][MW dwords]   activity bits of the whole tile (MW = BN/32)
//   tile   [BN cols][RS bytes]     rounded values of RPP rows, column-major
//   vals   [RPP][VS bytes]         slot values of each row of the pass
//   idxs   [RPP][IS bytes]         slot column offsets
//   dummy  [64][4 bytes]           where the lanes that hold no mask word write
template <Dt D, int BN>
struct EpilogueLds {
  using T = typename DtT<D>::T;
  static constexpr int S = (int)sizeof(T);
  static constexpr int MW = BN / 32;
  static constexpr int RPP = (BN * (128 * S + 8) <= 72 * 1024) ? 128 : 64;
  static constexpr int RS = RPP * S + 8;
  static constexpr int MASKS = GEMM_BM * MW * 4;
  static constexpr int TILE_OFF = MASKS;
  static constexpr int TILE = BN * RS;
  __host__ __device__ static constexpr int vs(int cap) { return (cap * S + 15) / 16 * 16; }
  __host__ __device__ static constexpr int is(int cap) { return (cap + 15) / 16 * 16; }
  __host__ __device__ static constexpr int vals_off() { return (TILE_OFF + TILE + 15) / 16 * 16; }
  __host__ __device__ static constexpr int idxs_off(int cap) { return vals_off() + RPP * vs(cap); }
  __host__ __device__ static constexpr int dummy_off(int cap) { return idxs_off(cap) + RPP * is(cap); }
  __host__ __device__ static constexpr int bytes(int cap) { return dummy_off(cap) + 64 * 4; }
};

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

// Copy `bytes` bytes LDS -> global in the widest unit both sides allow.
__device__ __forceinline__ void copy_out(char *__restrict__ g, const char *l, int bytes, int unit) {
  if (unit >= 16) {
    for (int o = 0; o < bytes; o += 16) *reinterpret_cast<u32x4_t *>(g + o) = *reinterpret_cast<const u32x4_t *>(l + o);
  } else if (unit >= 4) {
    for (int o = 0; o < bytes; o += 4) *reinterpret_cast<uint32_t *>(g + o) = *reinterpret_cast<const uint32_t *>(l + o);
  } else if (unit == 2) {
    for (int o = 0; o < bytes; o += 2) *reinterpret_cast<uint16_t *>(g + o) = *reinterpret_cast<const uint16_t *>(l + o);
  } else {
    for (int o = 0; o < bytes; ++o) g[o] = l[o];
  }
}

template <Dt D, int BN, bool DUMP>
__global__ __launch_bounds__(DMA_THREADS) void k_gate_twell(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wg,
    const float *__restrict__ beta, int M, int K, int N, int cap, uint16_t *__restrict__ cnt,
    typename DtT<D>::T *__restrict__ val, uint8_t *__restrict__ idx,
    typename DtT<D>::T *__restrict__ pre_out) {
  using T = typename DtT<D>::T;
  using WT = WaveTile<BN>;
  constexpr int NWM = WT::NWM, NWN = WT::NWN;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int mt = (M + GEMM_BM - 1) / GEMM_BM, ntl = N / BN;
  int tm, tn;
  tile_coords(blockIdx.x, mt, ntl, tm, tn);
  const int m0 = tm * GEMM_BM, n0 = tn * BN;
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
  gemm_mainloop_dma<D, BN>(acc, rowA, rowB, rowv, init, (int)(ldk / SLAB), smem);

  // ---- TwELL epilogue ----
  // M  every wave compares its accumulators with the activity threshold of the
  //    rounded value (v_cmp, one 64-bit mask per register: 32 columns of two
  //    rows) and files the masks in LDS as BN-bit row masks;
  // then per pass of RPP rows:
  //  V  the waves that own those rows stage the rounded values in LDS;
  //  C  one lane per row walks the row's set bits in ascending order (ffbl),
  //     puts the first `cap` (value, column) pairs in the row's LDS slots and
  //     writes count, slots and zero padding to global memory with vector
  //     stores.
  using L = EpilogueLds<D, BN>;
  constexpr int MW = L::MW, RPP = L::RPP, RS = L::RS, S = L::S;
  const int ntiles = N / BN;
  const int VS = L::vs(cap), IS = L::is(cap);
  char *tile = smem + L::TILE_OFF;
  char *vals = smem + L::vals_off();
  char *idxs = smem + L::idxs_off(cap);
  uint32_t *masks = reinterpret_cast<uint32_t *>(smem);
  const int vunit = (cap * S) % 16 == 0 ? 16 : ((cap * S) % 4 == 0 ? 4 : S);
  const int iunit = cap % 16 == 0 ? 16 : (cap % 4 == 0 ? 4 : 1);
  {
    // lane k < 2*NWN receives mask word col0/32 + k % NWN of row R (k < NWN)
    // or of row R+4
    const bool holder = lane < 2 * NWN;
    const int word = col0 / 32 + lane % NWN;
    const int roff = lane < NWN ? 0 : 4;
    uint32_t *dummy = reinterpret_cast<uint32_t *>(smem + L::dummy_off(cap)) + (tid & 63);
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
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
      }
    }
  }
  // The accumulators are read again by V: make them opaque here so that the
  // copies made for the masks are not kept live (which would spill).
#pragma unroll
  for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
    for (int bn = 0; bn < NWN; ++bn) asm volatile("" : "+a"(acc[bm][bn]));
#pragma unroll
  for (int p = 0; p < GEMM_BM / RPP; ++p) {
    // V: stage the rounded values of this pass and clear the slots
    for (int o = tid * 16; o < RPP * (VS + IS); o += DMA_THREADS * 16)
      *reinterpret_cast<u32x4_t *>(vals + o) = u32x4_t{0u, 0u, 0u, 0u};
    const int rl0 = row0 - p * RPP + 4 * (lane >> 5);  // lane's first row, relative to the pass
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm) {
      if ((row0 + 32 * bm) / RPP != p) continue;  // wave-uniform
#pragma unroll
      for (int bn = 0; bn < NWN; ++bn) {
        char *colp = tile + (col0 + 32 * bn + (lane & 31)) * RS;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          put4(colp + (rl0 + 32 * bm + 8 * g) * S, acc[bm][bn], 4 * g, T());
          if constexpr (DUMP) {
            const int t0 = m0 + p * RPP + rl0 + 32 * bm + 8 * g;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (t0 + q < M)
                pre_out[(size_t)(t0 + q) * N + n0 + col0 + 32 * bn + (lane & 31)] = from_f32<D>(acc[bm][bn][4 * g + q]);
          }
        }
      }
    }
    __syncthreads();
    // C: one lane per row
    if (lane < RPP / DMA_WAVES) {
      const int rl = wave * (RPP / DMA_WAVES) + lane;  // row within the pass
      const int rg = p * RPP + rl;                     // row within the tile
      const int t = m0 + rg;
      int n = 0, total = 0;
#pragma unroll
      for (int w = 0; w < MW; ++w) {
        uint32_t m = masks[rg * MW + w];
        total += __popc(m);
        while (m != 0 && n < cap) {
          const int c = 32 * w + __builtin_ctz(m);
          m &= m - 1;
          *reinterpret_cast<T *>(vals + rl * VS + n * S) = *reinterpret_cast<const T *>(tile + c * RS + rl * S);
          idxs[rl * IS + n] = (char)c;
          ++n;
        }
      }
      if (t < M) {
        const size_t slot0 = ((size_t)t * ntiles + tn) * cap;
        cnt[(size_t)t * ntiles + tn] = (uint16_t)total;
        copy_out(reinterpret_cast<char *>(val + slot0), vals + rl * VS, cap * S, vunit);
        copy_out(reinterpret_cast<char *>(idx + slot0), idxs + rl * IS, cap, iunit);
      }
    }
    __syncthreads();
  }
}

template <Dt D, int BN, bool DUMP>
static hipError_t launch_gate(const GateArgs &a, hipStream_t s) {
  using T = typename DtT<D>::T;
  auto kern = k_gate_twell<D, BN, DUMP>;
  const int lds = std::max(gemm_dma_lds_bytes(BN), EpilogueLds<D, BN>::bytes(64));
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int mt = (a.M + GEMM_BM - 1) / GEMM_BM, ntl = a.N / BN;
  hipLaunchKernelGGL(kern, dim3(mt * ntl), dim3(DMA_THREADS), lds, s, (const T *)a.x,
                     (const T *)a.wg, a.beta, a.M, a.K, a.N, a.cap, a.cnt, (T *)a.val, a.idx,
                     (T *)a.pre_out);
  return hipGetLastError();
}

template <Dt D, int BN>
static hipError_t launch_gate(const GateArgs &a, hipStream_t s) {
  return a.pre_out != nullptr ? launch_gate<D, BN, true>(a, s) : launch_gate<D, BN, false>(a, s);
}

hipError_t gate_twell(const GateArgs &a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.dtype == Dt::BF16) {
    if (a.tile == 256) return launch_gate<Dt::BF16, 256>(a, s);
    if (a.tile == 128) return launch_gate<Dt::BF16, 128>(a, s);
  } else {
    if (a.tile == 256) return launch_gate<Dt::F32, 256>(a, s);
    if (a.tile == 128) return launch_gate<Dt::F32, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace twell
