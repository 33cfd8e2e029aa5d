// MFMA GEMM mainloops for gfx950 shared by the gate, gate+up and down kernels.
//
// C[m][n] = sum_k A[m][k] * B(k, n), accumulated in fp32 on the matrix cores:
// bf16 operands use v_mfma_f32_32x32x16_bf16, fp32 operands v_mfma_f32_32x32x2_f32.
// The workgroup tile is BM = 256 rows x BN (128 or 256) columns.
//
// Two mainloops:
//  * gemm_mainloop_dma (A and B both K-contiguous: the gate and gate+up
//    matmuls): 8 waves, direct global -> LDS loads through a 4-stage ring,
//    described below.
//  * gemm_mainloop (B N-contiguous, W_d [F][d] in the down projection): 4
//    waves, register-staged loads with an in-register 8x8 transpose of B.
//    Wave w owns rows [64w, 64w + 64) and every column of the tile.  K is
//    consumed 128 bytes at a time (64 bf16 / 32 fp32); each stage keeps
//    A [256][128 B] and B [BN][128 B] in LDS, every 128-byte row is 8 chunks
//    of 16 bytes, and chunk c of row r sits at physical chunk c ^ ((r >> 1) & 7),
//    which makes the 16-lane phases of ds_read_b128 conflict-free on the
//    64-bank gfx950 LDS.  Two stages are double-buffered; the next stage's
//    global loads are issued before the current stage's MFMAs and written to
//    LDS after them.
#pragma once

#include "common.hpp"

#include <type_traits>

namespace twell {

constexpr int GEMM_BM = 256;
constexpr int GEMM_THREADS = 256;
constexpr int KCHUNK_BYTES = 128;  // K bytes per stage and LDS row

__host__ __device__ constexpr int gemm_lds_bytes(int bn) { return 2 * (GEMM_BM + bn) * KCHUNK_BYTES; }

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * KCHUNK_BYTES + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// ---- operand loaders -------------------------------------------------------
// Each loader moves one 128-byte K slab of its operand for the workgroup tile:
// issue(kt) reads global memory into registers, commit(dst) writes LDS.

// K-contiguous operand rows (A = activations; B = weight rows W[n][k]).
// Row r of the tile comes from row_ptr(r).  NR = rows in the tile.
template <int NR>
struct KRowLoader {
  static constexpr int PER_THREAD = NR * 8 / GEMM_THREADS;
  const char *ptr[PER_THREAD];
  u32x4_t reg[PER_THREAD];
  int row0, chunk;

  template <class RowPtr>
  __device__ __forceinline__ void init(int tid, RowPtr row_ptr) {
    row0 = tid >> 3;
    chunk = tid & 7;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) ptr[i] = row_ptr(row0 + 32 * i) + chunk * 16;
  }
  __device__ __forceinline__ void issue(int kt) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i)
      reg[i] = *reinterpret_cast<const u32x4_t *>(ptr[i] + (size_t)kt * KCHUNK_BYTES);
  }
  __device__ __forceinline__ void commit(char *dst) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i)
      *reinterpret_cast<u32x4_t *>(dst + lds_off(row0 + 32 * i, chunk)) = reg[i];
  }
};

// N-contiguous B operand (W[k][n] row-major, e.g. W_d [F][d] in the down
// projection): loaded as small k x n blocks and transposed in registers so
// that LDS holds the same [n][k] layout as a K-contiguous operand.
template <Dt D, int BN> struct NColLoader;

// bf16: 8 (k) x 8 (n) blocks, 16 bytes per k row; 8 x 8 transpose with v_perm.
// With fewer blocks than threads (BN = 128: 128 blocks) the first BLOCKS
// threads (whole waves) carry one block each and the others none.
template <int BN>
struct NColLoader<Dt::BF16, BN> {
  static constexpr int BLOCKS = BN / 8 * 8;  // (BN/8 n-blocks) x (8 k-blocks of 8)
  static constexpr int PER_THREAD = BLOCKS >= GEMM_THREADS ? BLOCKS / GEMM_THREADS : 1;
  static_assert(BLOCKS % 64 == 0, "whole waves of blocks");
  const char *base;
  size_t ld;  // bytes per k row
  int kb[PER_THREAD], nb[PER_THREAD];
  bool on;
  u32x4_t reg[PER_THREAD][8];

  __device__ __forceinline__ void init(int tid, const void *b, size_t ld_bytes, int n0) {
    ld = ld_bytes;
    base = reinterpret_cast<const char *>(b) + (size_t)n0 * 2;
    on = tid < BLOCKS;
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
      int blk = tid + GEMM_THREADS * p;
      kb[p] = blk & 7;
      nb[p] = blk >> 3;
    }
  }
  __device__ __forceinline__ void issue(int kt) {
    if (!on) return;
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
      const char *src = base + (size_t)(kt * 64 + kb[p] * 8) * ld + nb[p] * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) reg[p][i] = *reinterpret_cast<const u32x4_t *>(src + i * ld);
    }
  }
  __device__ __forceinline__ void commit(char *dst) {
    if (!on) return;
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // output row n = 8*nb + j holds k = 8*kb .. 8*kb+7: pair (k=2m, 2m+1) per dword
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t o;
        o.x = __builtin_amdgcn_perm(reg[p][1][j >> 1], reg[p][0][j >> 1], sel);
        o.y = __builtin_amdgcn_perm(reg[p][3][j >> 1], reg[p][2][j >> 1], sel);
        o.z = __builtin_amdgcn_perm(reg[p][5][j >> 1], reg[p][4][j >> 1], sel);
        o.w = __builtin_amdgcn_perm(reg[p][7][j >> 1], reg[p][6][j >> 1], sel);
        *reinterpret_cast<u32x4_t *>(dst + lds_off(nb[p] * 8 + j, kb[p])) = o;
      }
    }
  }
};

// fp32: 4 (k) x 4 (n) blocks; 4 x 4 transpose is a register renaming.
template <int BN>
struct NColLoader<Dt::F32, BN> {
  static constexpr int BLOCKS = BN / 4 * 8;
  static constexpr int PER_THREAD = BLOCKS / GEMM_THREADS;
  const char *base;
  size_t ld;
  int kb[PER_THREAD], nb[PER_THREAD];
  u32x4_t reg[PER_THREAD][4];

  __device__ __forceinline__ void init(int tid, const void *b, size_t ld_bytes, int n0) {
    ld = ld_bytes;
    base = reinterpret_cast<const char *>(b) + (size_t)n0 * 4;
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
      int blk = tid + GEMM_THREADS * p;
      kb[p] = blk & 7;
      nb[p] = blk >> 3;
    }
  }
  __device__ __forceinline__ void issue(int kt) {
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
      const char *src = base + (size_t)(kt * 32 + kb[p] * 4) * ld + nb[p] * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) reg[p][i] = *reinterpret_cast<const u32x4_t *>(src + i * ld);
    }
  }
  __device__ __forceinline__ void commit(char *dst) {
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t o = {reg[p][0][j], reg[p][1][j], reg[p][2][j], reg[p][3][j]};
        *reinterpret_cast<u32x4_t *>(dst + lds_off(nb[p] * 4 + j, kb[p])) = o;
      }
    }
  }
};

// ---- MFMA step ----------------------------------------------------------------

template <Dt D> struct Mfma;
template <> struct Mfma<Dt::BF16> {
  __device__ __forceinline__ static void step(f32x16_t &acc, const u32x4_t &a, const u32x4_t &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<Dt::F32> {
  // One 16-byte chunk per lane holds 4 k values; lanes 0-31 and 32-63 carry
  // different k, and A and B use the same assignment, so 4 rank-2 MFMAs cover
  // the 8 k values of the chunk pair.
  __device__ __forceinline__ static void step(f32x16_t &acc, const u32x4_t &a, const u32x4_t &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
  }
};

// Accumulate one LDS stage into acc[2][BN/32].
template <Dt D, int BN>
__device__ __forceinline__ void mfma_stage(f32x16_t (&acc)[2][BN / 32], const char *stage, int wave, int lane) {
  const char *As = stage;
  const char *Bs = stage + GEMM_BM * KCHUNK_BYTES;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x4_t a[2], b[BN / 32];
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
      a[bm] = *reinterpret_cast<const u32x4_t *>(As + lds_off(64 * wave + 32 * bm + r, 2 * g + h));
#pragma unroll
    for (int bn = 0; bn < BN / 32; ++bn)
      b[bn] = *reinterpret_cast<const u32x4_t *>(Bs + lds_off(32 * bn + r, 2 * g + h));
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < BN / 32; ++bn) Mfma<D>::step(acc[bm][bn], a[bm], b[bn]);
  }
}

// The double-buffered mainloop over nk K-slabs.
template <Dt D, int BN, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(f32x16_t (&acc)[2][BN / 32], LA &la, LB &lb, int nk, char *smem) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int STAGE = (GEMM_BM + BN) * KCHUNK_BYTES;
  la.issue(0);
  lb.issue(0);
  la.commit(smem);
  lb.commit(smem + GEMM_BM * KCHUNK_BYTES);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char *cur = smem + (kt & 1) * STAGE;
    char *nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      la.issue(kt + 1);
      lb.issue(kt + 1);
    }
    mfma_stage<D, BN>(acc, cur, wave, lane);
    if (more) {
      la.commit(nxt);
      lb.commit(nxt + GEMM_BM * KCHUNK_BYTES);
    }
    __syncthreads();
  }
}

// ---- mainloop with direct-to-LDS loads (k-contiguous operands) ------------
//
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight
// into LDS (M0 + 16 * lane), with no VGPR staging, so several stages can be in
// flight at once.  K is consumed in 64-byte slabs (32 bf16 / 16 fp32) through a
// ring of DMA_STAGES LDS stages that all start filled.  The loads are written
// as inline assembly and their completion is tracked with explicit s_waitcnt
// vmcnt: the compiler otherwise assumes every LDS read may alias an in-flight
// direct load and waits for all of them, which would serialise the ring.
//
// The workgroup has 8 waves (two per SIMD, so one wave's LDS reads overlap the
// other's MFMAs).  For BN = 256 the waves form a 2 x 4 grid of 128 x 64 wave
// tiles; for BN = 128 a 4 x 2 grid of 64 x 64.  A wave always spans 64 columns
// (two 32-column accumulator blocks) and WaveTile<BN>::NWM blocks of 32 rows.
// A wave's operand fragments are double-buffered in registers: the second
// half of slab kt is read from LDS while the first half is multiplied, and the
// first half of slab kt+1 while the second half of slab kt is multiplied.  One
// barrier per slab, placed after the last read of slab kt, frees its LDS stage
// for the loads of slab kt + DMA_STAGES.
//
// Each 64-byte LDS row holds 4 chunks of 16 bytes; chunk c of row r sits at
// physical chunk c ^ ((r >> 2) & 3), so the 16 lanes of one ds_read_b128 phase
// (16 consecutive rows, one chunk) hit 16 distinct 4-bank groups of the 64-bank
// LDS.

constexpr int SLAB = 64;  // K bytes per stage

// Shape of a DMA mainloop: BM rows per workgroup tile, WAVES waves, a ring of
// STAGES LDS stages.  Every wave owns 64 columns and BM / (WAVES / (BN / 64))
// rows of the tile.  DmaBig is the one in use: one workgroup per CU, 256 x BN
// tiles, 8 waves, 4 stages.  DmaHalf (two workgroups per CU, 128 x BN tiles, 4
// waves, 3 stages, so that one workgroup's epilogue overlaps the other's
// matrix-core work) gave bit-identical TwELL output but a slower gate matmul
// (265 against 240 us at the 1.5B-class shape): its smaller tiles move 1.5x
// the operand bytes per flop.
template <int BM_, int WAVES_, int STAGES_>
struct DmaCfg {
  static constexpr int BM = BM_, WAVES = WAVES_, THREADS = 64 * WAVES_, STAGES = STAGES_;
  // waves per SIMD the kernel must leave room for (register budget 512 / this)
  static constexpr int WAVES_PER_SIMD = 2;
  static_assert(STAGES == 3 || STAGES == 4, "the peeled tail covers 3- and 4-stage rings");
};
using DmaBig = DmaCfg<256, 8, 4>;
using DmaHalf = DmaCfg<128, 4, 3>;
constexpr int DMA_STAGES = DmaBig::STAGES;
constexpr int DMA_WAVES = DmaBig::WAVES;
constexpr int DMA_THREADS = DmaBig::THREADS;

// LDS: the ring, then one fp32 value per tile row (the gate bias, loaded with
// the first stages so that no separate global round trip delays the tile).
template <class Cfg = DmaBig>
__host__ __device__ constexpr int gemm_dma_ring_bytes(int bn) { return Cfg::STAGES * (Cfg::BM + bn) * SLAB; }
template <class Cfg = DmaBig>
__host__ __device__ constexpr int gemm_dma_lds_bytes(int bn) { return gemm_dma_ring_bytes<Cfg>(bn) + Cfg::BM * 4; }

template <int BN, class Cfg = DmaBig>
struct WaveTile {
  static constexpr int WPR = BN / 64;                                  // waves across the N tile
  static constexpr int NWN = 2;                                        // 32-column blocks per wave
  static constexpr int NWM = Cfg::BM / 32 / (Cfg::WAVES / WPR);        // 32-row blocks per wave
  static_assert(NWM >= 1 && Cfg::WAVES % WPR == 0, "whole waves across the tile");
  __device__ __forceinline__ static int row0(int wave) { return (wave / WPR) * 32 * NWM; }
  __device__ __forceinline__ static int col0(int wave) { return (wave % WPR) * 64; }
};

__device__ __forceinline__ int lds_off64(int row, int chunk) {
  return row * SLAB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char *)p);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One wave-wide 16-byte-per-lane copy global -> LDS [lds, lds + 1024).
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// One wave-wide 4-byte-per-lane copy global -> LDS [lds, lds + 256).
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n (0..3, wave-uniform) stages of OPS loads each are still
// in flight.
template <int OPS>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 3)
    wait_vmcnt<3 * OPS>();
  else if (n == 2)
    wait_vmcnt<2 * OPS>();
  else if (n == 1)
    wait_vmcnt<OPS>();
  else
    wait_vmcnt<0>();
}

// Rows of one operand tile loaded by DMA.  NR rows x 4 chunks = NR*4 lane
// slots = NR/16 wave instructions, spread over the WAVES waves.
template <int NR, int WAVES = DMA_WAVES>
struct DmaRows {
  static constexpr int PER_WAVE = NR / 16 / WAVES;  // instructions per wave per stage
  static_assert(PER_WAVE >= 1 && NR % (16 * WAVES) == 0, "whole 1 KB blocks per wave");
  const char *ptr[PER_WAVE];
  uint32_t lds_off[PER_WAVE];  // byte offset of the wave's 1 KB block in the stage

  template <class RowPtr>
  __device__ __forceinline__ void init(int wave_u, int lane, int region_off, RowPtr row_ptr) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave_u * PER_WAVE + j;  // 1 KB block = 16 rows
      const int row = blk * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      ptr[j] = row_ptr(row) + c * 16;
      lds_off[j] = region_off + blk * 1024;
    }
  }
  __device__ __forceinline__ void issue(int kt, uint32_t stage_base) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) dma16(ptr[j] + (size_t)kt * SLAB, stage_base + lds_off[j]);
  }
};

// Operand fragments of one 32-k half slab for a wave tile.
template <int NWM, int NWN>
struct Frag {
  u32x4_t a[NWM], b[NWN];
};

template <int BM, int NWM, int NWN>
__device__ __forceinline__ void read_frag(Frag<NWM, NWN> &f, const char *stage, int row0, int col0, int half,
                                          int lane) {
  const char *As = stage;
  const char *Bs = stage + BM * SLAB;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < NWM; ++i)
    f.a[i] = *reinterpret_cast<const u32x4_t *>(As + lds_off64(row0 + 32 * i + r, 2 * half + h));
#pragma unroll
  for (int j = 0; j < NWN; ++j)
    f.b[j] = *reinterpret_cast<const u32x4_t *>(Bs + lds_off64(col0 + 32 * j + r, 2 * half + h));
}

template <Dt D, int NWM, int NWN>
__device__ __forceinline__ void mfma_frag(f32x16_t (&acc)[NWM][NWN], const Frag<NWM, NWN> &f) {
#pragma unroll
  for (int i = 0; i < NWM; ++i)
#pragma unroll
    for (int j = 0; j < NWN; ++j) Mfma<D>::step(acc[i][j], f.a[i], f.b[j]);
}

// Mainloop over nk 64-byte K slabs; A rows from rowA(r), B rows from rowB(r).
// rowv(r) points at one fp32 value per tile row r (or is null for every r);
// those values are copied to LDS with the first stages, and init(acc, vals)
// sets the accumulators before the first MFMA, vals being the LDS copy
// (Cfg::BM floats) or null.
// The accumulators of one wave tile.
template <int BN, class Cfg>
using AccTile = f32x16_t[WaveTile<BN, Cfg>::NWM][WaveTile<BN, Cfg>::NWN];

template <Dt D, int BN, class Cfg, class RA, class RB, class RV, class INIT>
__device__ __forceinline__ void gemm_mainloop_dma(AccTile<BN, Cfg> &acc, RA rowA, RB rowB, RV rowv, INIT init,
                                                  int nk, char *smem) {
  using WT = WaveTile<BN, Cfg>;
  constexpr int BM = Cfg::BM, WAVES = Cfg::WAVES, STAGES = Cfg::STAGES;
  constexpr int NWM = WT::NWM, NWN = WT::NWN;
  constexpr int STAGE = (BM + BN) * SLAB;
  constexpr int OPS = DmaRows<BM, WAVES>::PER_WAVE + DmaRows<BN, WAVES>::PER_WAVE;  // DMA ops per stage per lane
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = WT::row0(wave_u), col0 = WT::col0(wave_u);
  const uint32_t base = lds_address(smem);
  const bool has_rowv = rowv(0) != nullptr;
  DmaRows<BM, WAVES> da;
  DmaRows<BN, WAVES> db;
  da.init(wave_u, lane, 0, rowA);
  db.init(wave_u, lane, BM * SLAB, rowB);
  // BM / 64 waves copy 64 row values each; issued before the stages, so the
  // stage waits below cover them (loads complete in order)
  if (has_rowv && wave_u < BM / 64)
    dma4(rowv(64 * wave_u + lane), base + gemm_dma_ring_bytes<Cfg>(BN) + 256 * wave_u);
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    if (s < nk) {
      da.issue(s, base + s * STAGE);
      db.issue(s, base + s * STAGE);
    }
  }
  wait_stages<OPS>(min(nk - 1, STAGES - 1));
  __syncthreads();
  init(acc, has_rowv ? reinterpret_cast<const float *>(smem + gemm_dma_ring_bytes<Cfg>(BN)) : nullptr);
  Frag<NWM, NWN> f0, f1;
  read_frag<BM>(f0, smem, row0, col0, 0, lane);
  // One slab kt < nk - 1 with WAIT stages (of OPS loads) left in flight at its
  // barrier, issuing the loads of slab kt + STAGES if ISSUE.  The loop is
  // peeled by these constants (no runtime selection of the wait) and the last
  // slab has a block of its own: a path that joins the steady state with the
  // last slab's makes the compiler wait for the next slab's first-half reads
  // before the second-half MFMAs.
  auto slab = [&](auto wait_c, auto issue_c, int kt) {
    constexpr int WAIT = decltype(wait_c)::value;
    constexpr bool ISSUE = decltype(issue_c)::value;
    const int slot = kt % STAGES;
    read_frag<BM>(f1, smem + slot * STAGE, row0, col0, 1, lane);
    mfma_frag<D>(acc, f0);
    // Scheduling hint: alternate the MFMAs of the first half with the LDS
    // reads of the second, one each, instead of issuing the reads in a block.
#pragma unroll
    for (int q = 0; q < NWM + NWN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    // every wave has read all of slab kt (the barrier waits for its LDS
    // reads) and slab kt+1 has landed for every wave
    wait_vmcnt<WAIT * OPS>();
    __syncthreads();
    if constexpr (ISSUE) {
      const uint32_t sb = base + slot * STAGE;
      da.issue(kt + STAGES, sb);
      db.issue(kt + STAGES, sb);
    }
    read_frag<BM>(f0, smem + ((kt + 1) % STAGES) * STAGE, row0, col0, 0, lane);
    mfma_frag<D>(acc, f1);
    // the same alternation for the next slab's first-half reads
#pragma unroll
    for (int q = 0; q < NWM + NWN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using IW = std::integral_constant<int, STAGES - 2>;
  using BT = std::integral_constant<bool, true>;
  using BF = std::integral_constant<bool, false>;
  // slab kt waits for slab kt + 1: min(nk - 2 - kt, STAGES - 2) stages stay in
  // flight; slab kt + STAGES is loaded while kt + STAGES < nk
  int kt = 0;
  for (; kt + STAGES < nk; ++kt) slab(IW(), BT(), kt);
  if constexpr (STAGES == 4) {
    if (kt == nk - 4) slab(I2(), BF(), kt++);
  }
  if (kt == nk - 3) slab(I1(), BF(), kt++);
  if (kt == nk - 2) slab(I0(), BF(), kt++);
  // the last slab: both halves, no loads left
  read_frag<BM>(f1, smem + (kt % STAGES) * STAGE, row0, col0, 1, lane);
  mfma_frag<D>(acc, f0);
  mfma_frag<D>(acc, f1);
  // no DMA is left in flight; make every wave's last LDS reads complete before
  // the caller reuses LDS
  __syncthreads();
}

// Accumulator element (bm, bn, i) of lane l sits at tile row
//   row0 + 32*bm + 8*(i/4) + 4*(l/32) + (i%4)   and tile column col0 + 32*bn + (l%32),
// with (row0, col0) the origin of the wave's tile (64 * wave, 0 in the 4-wave
// register-staged mainloop).
__device__ __forceinline__ int acc_row(int row0, int bm, int i, int lane) {
  return row0 + 32 * bm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Grouped, XCD-aware order of (m-tile, n-tile) pairs: the tiles that run at the
// same time on one XCD share GROUP_M row panels of A and a run of B panels.
__device__ __forceinline__ void tile_coords(int bid, int mt, int nt, int &tm, int &tn) {
  const int total = mt * nt;
  const int L = xcd_linear(bid, total);
  constexpr int GROUP_M = 4;
  const int per_group = GROUP_M * nt;
  const int g = L / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(GROUP_M, mt - first_m);
  const int in = L - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace twell
