// Gate matmul with the TwELL epilogue.
//
// pre[t][j] = sum_k x[t][k] * w_gate[j][k] + beta[t] on the matrix cores; the
// epilogue rounds every value to the storage dtype, applies ReLU and writes
// the TwELL matrix of the tile straight from the accumulator registers.  This
// is the "sparsity materialised in the epilogue of the dense matmul, no
// separate conversion pass and no synchronisation between workgroups" design
// of gist.science "Sparser, Faster, Lighter Transformer Language Models",
// Resumen Técnico §2.A, carried over to gfx950: the N tile of the matmul is
// exactly one TwELL tile and one wave holds whole tile rows, so counts, ranks
// and slot positions come from wave ballots (v_cmp masks) and mbcnt prefix
// counts with no LDS round trip and no inter-wave exchange.
#include "gemm.hpp"
#include "launch.hpp"

namespace twell {

template <Dt D, int BN>
__global__ __launch_bounds__(GEMM_THREADS) void k_gate_twell(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wg,
    const float *__restrict__ beta, int M, int K, int N, int cap, uint16_t *__restrict__ cnt,
    typename DtT<D>::T *__restrict__ val, uint8_t *__restrict__ idx,
    typename DtT<D>::T *__restrict__ pre_out) {
  using T = typename DtT<D>::T;
  constexpr int NB = BN / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int mt = (M + GEMM_BM - 1) / GEMM_BM, ntl = N / BN;
  int tm, tn;
  tile_coords(blockIdx.x, mt, ntl, tm, tn);
  const int m0 = tm * GEMM_BM, n0 = tn * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t ldk = (size_t)K * sizeof(T);

  KRowLoader<GEMM_BM> la;
  la.init(tid, [&](int r) {
    int row = min(m0 + r, M - 1);
    return reinterpret_cast<const char *>(x) + (size_t)row * ldk;
  });
  KRowLoader<BN> lb;
  lb.init(tid, [&](int r) { return reinterpret_cast<const char *>(wg) + (size_t)(n0 + r) * ldk; });

  // The accumulators start at beta so that the matmul adds the gate bias.
  f32x16_t acc[2][NB];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
    f32x16_t b0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int t = m0 + acc_row(wave, bm, i, lane);
      b0[i] = (beta != nullptr && t < M) ? beta[t] : 0.0f;
    }
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) acc[bm][bn] = b0;
  }

  gemm_mainloop<D, BN>(acc, la, lb, K / (KCHUNK_BYTES / (int)sizeof(T)), smem);

  // ---- TwELL epilogue ----
  const int ntiles = N / BN;
  const int col = lane & 31;
  const bool hi = lane >= 32;
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = m0 + acc_row(wave, bm, i, lane);
      const bool row_ok = t < M;
      const size_t slot0 = ((size_t)t * ntiles + tn) * cap;
      int base_lo = 0, base_hi = 0;  // active entries already placed in the two rows
#pragma unroll
      for (int bn = 0; bn < NB; ++bn) {
        const float v = acc[bm][bn][i];
        const bool act = active_after_round<D>(v) && row_ok;
        if (pre_out != nullptr && row_ok)
          pre_out[(size_t)t * N + n0 + 32 * bn + col] = from_f32<D>(v);
        const uint64_t m = ballot(act);
        if (m != 0) {
          const int n_lo = __popc((uint32_t)m), n_hi = __popc((uint32_t)(m >> 32));
          const int rank = mbcnt(m) - (hi ? n_lo : 0) + (hi ? base_hi : base_lo);
          if (act && rank < cap) {
            val[slot0 + rank] = from_f32<D>(v);
            idx[slot0 + rank] = (uint8_t)(32 * bn + col);
          }
          base_lo += n_lo;
          base_hi += n_hi;
        }
      }
      if (row_ok) {
        const int c = hi ? base_hi : base_lo;
        if (col == 0) cnt[(size_t)t * ntiles + tn] = (uint16_t)c;
        for (int s = col; s < cap; s += 32) {
          if (s >= c) {
            val[slot0 + s] = T(0);
            idx[slot0 + s] = 0;
          }
        }
      }
    }
  }
}

template <Dt D, int BN>
static hipError_t launch_gate(const GateArgs &a, hipStream_t s) {
  using T = typename DtT<D>::T;
  auto kern = k_gate_twell<D, BN>;
  const int lds = gemm_lds_bytes(BN);
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int mt = (a.M + GEMM_BM - 1) / GEMM_BM, ntl = a.N / BN;
  hipLaunchKernelGGL(kern, dim3(mt * ntl), dim3(GEMM_THREADS), lds, s, (const T *)a.x,
                     (const T *)a.wg, a.beta, a.M, a.K, a.N, a.cap, a.cnt, (T *)a.val, a.idx,
                     (T *)a.pre_out);
  return hipGetLastError();
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
