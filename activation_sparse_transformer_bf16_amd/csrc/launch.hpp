// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.hpp"

namespace twell {

// Gate matmul + TwELL epilogue (tile == matmul N tile).
struct GateArgs {
  Dt dtype;
  int tile;
  const void *x;      // [M][K]
  const void *wg;     // [N][K]
  const float *beta;  // [M] or null
  int M, K, N, cap;
  uint16_t *cnt;      // [M][N/tile]
  void *val;          // [M][N/tile][cap]
  uint8_t *idx;       // [M][N/tile][cap]
  void *pre_out;      // [M][N] or null
  bool tile_major = false;  // records at k * M + t instead of t * (N/tile) + k
};
hipError_t gate_twell(const GateArgs &a, hipStream_t s);

// Overflow scan: row flags, ascending overflow row list, its true length.
struct ScanArgs {
  const uint16_t *cnt;  // [T][nt]
  int T, nt, cap;
  uint8_t *row_flag;    // [T] or null
  int *ovf_rows;        // [ovf_cap] (may be null when ovf_cap == 0)
  int ovf_cap;
  int *n_ovf;           // [1]
  bool tile_major = false;  // cnt is [nt][T]
};
hipError_t overflow_scan(const ScanArgs &a, hipStream_t s);

// Ascending list of the rows with row_flag[t] != 0, and its true length.
hipError_t compact_rows(const uint8_t *row_flag, int T, int *ovf_rows, int ovf_cap, int *n_ovf, hipStream_t s);
// The same from int32 flags [T], listing the rows over the flag array itself.
hipError_t compact_rows_in_place(int *flags_then_rows, int T, int *n_ovf, hipStream_t s);

// How the up projection cuts its weights: hidden units in groups of tpg
// TwELL tiles (about 4 MB of W_u^T rows, one XCD's L2), and, when the groups
// need more than one round over the 8 XCDs, each W_u^T row in dc = 2 halves
// of d (a group then holds twice the units, so x is streamed half as often;
// the halves' partial dot products meet in a 16-byte list entry).
struct UpPlan {
  int tpg, n_groups, dc;
  int entry_bytes() const { return dc == 1 ? 8 : 16; }
};
constexpr int UP_LIST = 256;  // entries per wave list (tiles per group * cap)
inline UpPlan up_plan(int d, int F, int tile, int cap, Dt dt) {
  const int s = dt == Dt::BF16 ? 2 : 4;
  const int nt = F / tile;
  const size_t group_target = (size_t)4 << 20;
  auto tiles_per_group = [&](int dc) {
    const size_t tile_bytes = (size_t)tile * (d / dc) * s;
    int tpg = (int)std::max<size_t>(1, group_target / tile_bytes);
    tpg = std::min(tpg, std::min(std::min(64, nt), UP_LIST / cap));
    while (nt % tpg != 0) --tpg;
    return tpg;
  };
  UpPlan p{tiles_per_group(1), 0, 1};
  p.n_groups = nt / p.tpg;
  // a half row must still cover whole 16-byte chunks of all 64 lanes
  if (p.n_groups > 8 && (d / 2) % (64 * (16 / s)) == 0) {
    p.dc = 2;
    p.tpg = tiles_per_group(2);
    p.n_groups = nt / p.tpg;
  }
  return p;
}

// Sparse up / down projections over the TwELL entries of non-overflow rows.
// Each compact entry list is padded to a multiple of LIST_PAD entries (the
// down projection consumes up to LIST_PAD entries per step without a bound
// check on the list length).
constexpr int LIST_PAD = 16;

struct SparseArgs {
  Dt dtype;
  int T, d, F, tile, cap;
  const uint16_t *cnt;
  const void *val;
  const uint8_t *idx;
  uint8_t *row_flag;        // [T], written by the up kernel: 1 = overflow row (dense fallback)
  const void *x;            // [T][d]
  const void *wu;           // [F][d]
  const void *wd;           // [F][d]
  void *list;               // [T][stride] entries: UpPlan dc == 1: (uint32 row byte offset, v = round(h * u));
                            // dc == 2: (offset, fp32 partial u of the first half of d, fp32 h, partial of the second)
  int *list_n;              // [T] entries per row
  int stride;               // list entries per row: nt * cap rounded up to a multiple of LIST_PAD
  void *y;                  // [T][d]
  float *u = nullptr;       // [T][nt][cap] saved u per TwELL slot (NaN for overflow rows), or null
  bool tile_major = false;  // TwELL records tile-major (read by the grouped fused kernel only)
};
hipError_t sparse_up(const SparseArgs &a, hipStream_t s);
hipError_t sparse_down(const SparseArgs &a, hipStream_t s);
// Up and down in one kernel (one wave per token); writes row_flag and the y
// rows of non-overflow tokens; list / list_n / stride are not used.
hipError_t sparse_fused(const SparseArgs &a, hipStream_t s);

// The hidden-group-major variant: groups of tpg TwELL tiles whose W_u and W_d
// rows together are about 4 MB (one XCD's L2), at most 16 groups; partial
// output rows [n_groups][T][d] fp32, added in group order by a second kernel.
struct FusedGroups {
  int tpg, n_groups;
};
inline FusedGroups fused_groups(int d, int F, int tile, Dt dt) {
  const int s = dt == Dt::BF16 ? 2 : 4;
  const int nt = F / tile;
  const size_t tile_bytes = (size_t)2 * tile * d * s;  // W_u and W_d rows of one tile
  int tpg = (int)std::max<size_t>(1, ((size_t)4 << 20) / tile_bytes);
  tpg = std::max(tpg, (nt + 15) / 16);
  tpg = std::min(tpg, nt);
  return FusedGroups{tpg, (nt + tpg - 1) / tpg};
}
hipError_t sparse_fused_grouped(const SparseArgs &a, float *partial, hipStream_t s);

// Dense ReGLU FFN on the matrix cores over a (possibly gathered) set of rows:
// logical row r < n_rows reads x[rows ? rows[r] : r] and writes y at the same
// physical row.  With n_rows_dev (device int) non-null the row count is
// clamp(*n_rows_dev - n_sub, 0, M): one chunk of M rows of a longer list whose
// first n_sub rows earlier chunks took; the grid is sized for M and
// workgroups past the device count exit at once.
struct DenseArgs {
  Dt dtype;
  const void *x, *wg, *wu, *wd;
  const float *beta;   // indexed by physical row, or null
  void *y;             // [T][d]
  int M, d, F;         // M = grid rows (T, or the chunk's rows)
  const int *rows;     // [M] or null (identity)
  const int *n_rows_dev;
  int n_sub;           // rows of *n_rows_dev taken by earlier chunks
  void *a_ws;          // [M][F] storage dtype, logical rows
  void *h_out;         // [h_cap][F] storage dtype (ReLU'd gate rows) or null
  int h_cap;
  float *partial;      // fallback only: split-K partial tiles (partial_tiles of FALLBACK_SPLIT_TILE floats)
  int partial_tiles;   // capacity of `partial` in tiles; 0 = no split
};

// The fallback's split-K.  Its grid has FALLBACK_WGS workgroups; when the
// rows fill fewer output tiles than that, K is cut into S ranges whose fp32
// partial tiles (256 x 256) a reduction kernel adds in K order.  S is at most
// smax, at most the K slabs nk, and S * tiles stays within the capacity of
// the partial area.
constexpr int FALLBACK_WGS = 256;
constexpr int FALLBACK_SPLIT_TILE = 256 * 256;  // floats of one partial tile
constexpr int GATE_UP_SPLIT_MAX = 2;
constexpr int DOWN_SPLIT_MAX = 16;
constexpr int FALLBACK_PARTIAL_TILES_MAX = 128;  // 32 MB of partial tiles at most
constexpr int FALLBACK_DOWN_BN = 128;            // output columns per tile of the fallback's down matmul
__host__ __device__ inline int fallback_split(int tiles, int nk, int smax, int cap_tiles) {
  const int t = tiles > 0 ? tiles : 1;
  int s = FALLBACK_WGS / t;
  s = s < smax ? s : smax;
  s = s < nk ? s : nk;
  s = s < cap_tiles / t ? s : cap_tiles / t;
  return s > 1 ? s : 1;
}
hipError_t dense_gate_up(const DenseArgs &a, hipStream_t s);
hipError_t dense_down(const DenseArgs &a, hipStream_t s);

// Standalone TwELL packing of an explicit pre-activation matrix.
struct PackArgs {
  Dt dtype;
  int tile, cap;
  const void *pre;  // [T][F]
  int T, F;
  uint16_t *cnt;
  void *val;
  uint8_t *idx;
  int *row_flag;  // [T] int32: 1 for an overflowing row, else 0; or null
};
hipError_t pack_tiles(const PackArgs &a, hipStream_t s);

// dense[r] = ReLU(pre[ovf_rows[r]]) for r < min(*n_ovf, ovf_cap).
struct DenseRowsArgs {
  Dt dtype;
  const void *pre;
  int T, F;
  const int *ovf_rows;
  const int *n_ovf;
  int ovf_cap;
  void *dense;
};
hipError_t pack_dense_rows(const DenseRowsArgs &a, hipStream_t s);

// TwELL -> hybrid (ELL rows of `width` slots + dense backup rows).
struct HybridArgs {
  Dt dtype;
  int T, F, tile, cap;
  const uint16_t *cnt;   // TwELL
  const void *val;
  const uint8_t *idx;
  const int *ovf_rows;
  const int *n_ovf;
  int ovf_cap;
  const void *tw_dense;  // [ovf_cap][F] ReLU'd TwELL overflow rows
  int width;             // hybrid
  int *out_cnt;          // [T]
  void *out_val;         // [T][width]
  int *out_col;          // [T][width]
  int *dense_rows;       // [dense_cap]
  int *n_dense;          // [1]
  int dense_cap;
  void *out_dense;       // [dense_cap][F] or null
  const float *tw_u = nullptr;  // TwELL saved u [T][F/tile][cap], or null
  float *out_u = nullptr;       // hybrid saved u [T][width], or null
};
hipError_t twell_to_hybrid_launch(const HybridArgs &a, hipStream_t s);

// L1 activation penalty from TwELL: ||h||_1 (float64, deterministic) and the
// gradient lam * [h > 0] in the TwELL pattern.
constexpr int L1_BLOCKS = 1024;
struct L1Args {
  Dt dtype;
  int T, F, tile, cap;
  const uint16_t *cnt;
  const void *val;
  const int *n_ovf;
  int ovf_cap;
  const void *dense;   // [ovf_cap][F] ReLU'd overflow rows
  double *partial;     // [L1_BLOCKS] workspace (norm)
  double *out;         // [1] (norm)
  float lam;           // (gradient)
  void *grad_val;      // [T][F/tile][cap] (gradient)
  void *grad_dense;    // [ovf_cap][F] or null (gradient)
};
hipError_t l1_norm(const L1Args &a, hipStream_t s);
hipError_t l1_grad(const L1Args &a, hipStream_t s);

// FFN backward from hybrid activations: dx (activation dtype) and dW_g,
// dW_u, dW_d (fp32, [F][d]).  Workspace pieces: dcol/dn (compacted dense
// rows), ent (du, dpre per entry slot), pos (column-major place of each
// entry), csc (column-major records t, a, du, dpre), blk/boff/tot/colptr
// (the transpose's counts and offsets).
struct BackwardArgs {
  Dt dtype;
  int T, d, F, width;
  const int *cnt;
  const void *val;
  const int *col;
  const int *dense_rows;
  const int *n_dense;
  int dense_cap;
  const void *dense;
  const void *x, *dy, *wg, *wu, *wd;
  float lam;
  void *dx;
  float *dwg, *dwu, *dwd;
  int *dcol, *dn;
  void *ent;
  int *pos;
  void *csc;
  uint8_t *blk;
  int *boff, *tot, *colptr;
  int *order;  // [T] row order of the per-row kernels
  // The dense backup rows on the matrix cores (dense_mma; F a multiple of
  // 128).  Otherwise their entries are walked like the others (dcol / dn) and
  // these are null.  rcp = dense_cap rounded up to whole K chunks
  // (backward_dense_rows_padded), ns = 2 parts per value for bf16, 1 for fp32.
  bool dense_mma;
  void *bd_xr, *bd_dyr;            // [ns * rcp][d] gathered x / dy rows
  void *bd_du, *bd_dp;             // [dense_cap][F] du, dpre (storage dtype)
  void *bd_at, *bd_dut, *bd_dpt;   // [F][ns * rcp] a, du, dpre transposed (bf16: high, then low parts)
  float *bd_part;                  // dx split-K partial tiles
  int bd_part_tiles;               // their capacity in 256 x 256 fp32 tiles
  const float *u = nullptr;        // hybrid's saved u [T][width] or null
};
hipError_t ffn_backward(const BackwardArgs &a, hipStream_t s);
// The dense rows' part, launched by ffn_backward: their dx rows (U, DA, and
// the dx matmul) after the entry kernels' dx, their weight-gradient part
// before the entry kernels' weight gradients, which add onto it.
hipError_t ffn_backward_dense_dx(const BackwardArgs &a, hipStream_t s);
hipError_t ffn_backward_dense_dw(const BackwardArgs &a, hipStream_t s);
int backward_dense_partial_tiles(int dense_cap, int d);
int backward_dense_rows_padded(int dense_cap, Dt dt);

// *p = 0 with a one-thread kernel (safe under stream capture).
hipError_t zero_int(int *p, hipStream_t s);

// Streaming HBM probe: mode 0 reads `bytes` from src (dst: a 4-byte sink),
// mode 1 copies them to dst.
hipError_t stream_probe(const void *src, void *dst, size_t bytes, int mode, hipStream_t s);

// Matrix-core probe: `blocks` workgroups of 8 waves, each wave `iters` rounds
// of 8 independent 32x32x16 bf16 MFMAs on registers.
hipError_t mfma_probe(float *sink, int iters, int blocks, hipStream_t s);

}  // namespace twell
