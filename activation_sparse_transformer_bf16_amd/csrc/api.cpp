// C ABI of libtwell.so: argument validation, workspace layout and the launch
// sequence of every entry point declared in include/twell.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "twell.h"

using namespace twell;

namespace {

thread_local char g_err[512] = "";

void set_err(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

twell_status fail(twell_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

twell_status hip_check(hipError_t e, const char *what) {
  if (e == hipSuccess) return TWELL_OK;
  set_err("%s: %s", what, hipGetErrorString(e));
  return TWELL_ERR_HIP;
}

#define TW_TRY(expr, what)                           \
  do {                                               \
    twell_status st_ = hip_check((expr), (what));    \
    if (st_ != TWELL_OK) return st_;                 \
  } while (0)

constexpr size_t ALIGN_WS = 256;
constexpr int GEMM_ROWS = 256;  // rows of one fallback matmul tile

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int dt_size(twell_dtype dt) { return dt == TWELL_BF16 ? 2 : 4; }

Dt to_dt(twell_dtype dt) { return dt == TWELL_BF16 ? Dt::BF16 : Dt::F32; }

bool valid_dtype(int dt) { return dt == TWELL_F32 || dt == TWELL_BF16; }

// Format parameters shared by every entry point.
twell_status check_format(int tile, int cap, int F, int dtype) {
  if (!valid_dtype(dtype)) return fail(TWELL_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (tile <= 0 || F <= 0 || cap <= 0) return fail(TWELL_ERR_INVALID_ARG, "tile, cols and cap must be positive");
  if (F % tile != 0) return fail(TWELL_ERR_INVALID_ARG, "cols (%d) must be a multiple of the tile (%d)", F, tile);
  if (tile != 128 && tile != 256) return fail(TWELL_ERR_UNSUPPORTED, "tile %d not built (128 or 256)", tile);
  if (cap > std::min(tile, 64)) return fail(TWELL_ERR_UNSUPPORTED, "cap %d not built (1..%d)", cap, std::min(tile, 64));
  if (F > (1 << 24)) return fail(TWELL_ERR_UNSUPPORTED, "cols %d too large", F);
  return TWELL_OK;
}

twell_status check_d(int d, int dtype) {
  if (d <= 0) return fail(TWELL_ERR_INVALID_ARG, "d must be positive");
  // one row of x is held in registers as at most 16 16-byte chunks per lane
  const int q = dtype == TWELL_BF16 ? 512 : 256;
  if (d % q != 0 || d > 16 * q)
    return fail(TWELL_ERR_UNSUPPORTED, "d %d not built (multiple of %d, <= %d)", d, q, 16 * q);
  return TWELL_OK;
}

// The gather kernels address weight rows with 32-bit byte offsets.
twell_status check_weight_bytes(int F, int d, int dtype) {
  if ((size_t)F * (size_t)d * (size_t)dt_size((twell_dtype)dtype) >= ((size_t)1 << 31))
    return fail(TWELL_ERR_UNSUPPORTED, "weight matrices of F*d = %zu elements are too large", (size_t)F * d);
  return TWELL_OK;
}

twell_status check_matrix(const twell_matrix *m, bool need_ovf_all) {
  if (m == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null twell_matrix");
  if (m->rows < 0) return fail(TWELL_ERR_INVALID_ARG, "rows must be >= 0");
  if (m->ovf_cap < 0) return fail(TWELL_ERR_INVALID_ARG, "ovf_cap must be >= 0");
  twell_status st = check_format(m->tile, m->cap, m->cols, (int)m->dtype);
  if (st != TWELL_OK) return st;
  if (m->n_ovf == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null n_ovf");
  if (m->rows > 0 && (m->cnt == nullptr || m->val == nullptr || m->idx == nullptr))
    return fail(TWELL_ERR_INVALID_ARG, "null cnt/val/idx");
  if (m->ovf_cap > 0 && m->ovf_rows == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null ovf_rows with ovf_cap > 0");
  if (need_ovf_all && m->ovf_cap < m->rows)
    return fail(TWELL_ERR_INVALID_ARG, "ovf_cap (%d) must be >= rows (%d)", m->ovf_cap, m->rows);
  if (!aligned(m->cnt, 2) || !aligned(m->val, dt_size(m->dtype)) || !aligned(m->ovf_rows, 4) ||
      !aligned(m->n_ovf, 4) || !aligned(m->dense, 16) || !aligned(m->u, 4))
    return fail(TWELL_ERR_UNSUPPORTED, "misaligned twell_matrix buffer");
  if (m->layout != TWELL_LAYOUT_ROWS && m->layout != TWELL_LAYOUT_TILES)
    return fail(TWELL_ERR_INVALID_ARG, "unknown layout %d", (int)m->layout);
  if (m->layout == TWELL_LAYOUT_TILES && m->u != nullptr)
    return fail(TWELL_ERR_INVALID_ARG, "a tile-major TwELL matrix carries no u (packed->u must be NULL)");
  return TWELL_OK;
}

// Entry points that read or write the row-major layout only.
twell_status check_rows_layout(const twell_matrix *m, const char *who) {
  if (m->layout != TWELL_LAYOUT_ROWS)
    return fail(TWELL_ERR_UNSUPPORTED, "%s takes the row-major TwELL layout only", who);
  return TWELL_OK;
}

// Producers of a TwELL matrix that do not compute u take u == NULL.
twell_status check_no_u(const twell_matrix *m, const char *who) {
  if (m->u != nullptr) return fail(TWELL_ERR_INVALID_ARG, "%s does not save u: packed->u must be NULL", who);
  return TWELL_OK;
}

// Workspace of the sparse forward:
//   row flags [T] u8 | entry counts [T] i32 |
//   region A: the compact entry lists [T][stride] x 8 bytes (16 when the up
//             projection splits d in two halves, see UpPlan), and afterwards
//             (the lists are consumed by the down projection before the
//             fallback starts, in stream order) the fallback's activations
//             [R][F] in the storage dtype for one chunk of R overflow rows |
//   the fallback's split-K partial tiles (only as many as a split can use).
// The fallback takes the overflow rows R at a time, so the workspace stays
// below the dense [T][F] activation matrix it replaces.
struct FfnWs {
  size_t flag, list_n, list, a, partial, total;
  int stride, chunk_rows, partial_tiles;
};

// Rows per fallback chunk: half the batch (rounded up to 256 rows), all of
// it for T <= 512; so the common case (few or no overflow rows) is one chunk
// and the worst case (every row overflows) two.
int default_chunk_rows(int T) {
  const int half = (T + 1) / 2;
  return std::max(1, std::min(T, (half + 255) / 256 * 256));
}

// The largest number of partial tiles the fallback's split-K can use with
// chunks of R rows and an area of at most cap_tiles tiles (the device picks S
// with the same fallback_split, given the area's capacity).
int fallback_partial_tiles(int R, int d, int F, twell_dtype dt, int cap_tiles) {
  const int s = dt_size(dt);
  const int row_tiles = (R + GEMM_ROWS - 1) / GEMM_ROWS;
  const int nk_gu = d * s / 64, ntl_gu = F / 128;                 // gate+up: 64-byte K slabs, 128-unit tiles
  const int nk_dn = F * s / 128, ntl_dn = d / FALLBACK_DOWN_BN;   // down: 128-byte K chunks
  const int per = 256 / FALLBACK_DOWN_BN;                         // down partial tiles per 256 x 256 tile
  int best = 0;
  for (int rt = 1; rt <= row_tiles; ++rt) {
    const int tg = rt * ntl_gu, td = rt * ntl_dn;
    const int sg = fallback_split(tg, nk_gu, GATE_UP_SPLIT_MAX, cap_tiles);
    const int sd = fallback_split(td, nk_dn, DOWN_SPLIT_MAX, cap_tiles * per);
    if (sg > 1) best = std::max(best, sg * tg);
    if (sd > 1) best = std::max(best, (sd * td + per - 1) / per);
  }
  return best;
}

FfnWs ffn_ws_layout(int T, int d, int F, int tile, int cap, twell_dtype dt, int chunk_rows,
                    int partial_cap = FALLBACK_PARTIAL_TILES_MAX) {
  FfnWs w;
  const size_t nt = (size_t)F / tile;
  w.stride = (int)((nt * cap + LIST_PAD - 1) / LIST_PAD * LIST_PAD);
  w.chunk_rows = chunk_rows;
  w.partial_tiles = T > 0 ? fallback_partial_tiles(chunk_rows, d, F, dt, partial_cap) : 0;
  w.flag = 0;
  w.list_n = align_up((size_t)T, ALIGN_WS);
  w.list = align_up(w.list_n + (size_t)T * 4, ALIGN_WS);
  w.a = w.list;  // aliases the lists (see above)
  const size_t entry = (size_t)up_plan(d, F, tile, cap, to_dt(dt)).entry_bytes();
  const size_t region = std::max((size_t)T * w.stride * entry, (size_t)chunk_rows * F * dt_size(dt));
  w.partial = align_up(w.list + region, ALIGN_WS);
  w.total = std::max(align_up(w.partial + (size_t)w.partial_tiles * FALLBACK_SPLIT_TILE * 4, ALIGN_WS), ALIGN_WS);
  return w;
}

FfnWs ffn_ws_layout(int T, int d, int F, int tile, int cap, twell_dtype dt) {
  return ffn_ws_layout(T, d, F, tile, cap, dt, default_chunk_rows(T));
}

twell_status check_ffn_ptrs(const void *x, const void *wg, const void *wu, const void *wd, const float *beta,
                            const void *y) {
  if (!x || !wg || !wu || !wd || !y) return fail(TWELL_ERR_INVALID_ARG, "null x/w_gate/w_up/w_down/y");
  if (!aligned(x, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) || !aligned(y, 16) ||
      !aligned(beta, 4))
    return fail(TWELL_ERR_UNSUPPORTED, "x, weights and y must be 16-byte aligned");
  return TWELL_OK;
}

// The overflow-row list, then the dense fallback over it, chunk by chunk.
// Chunk c takes list positions [c R, c R + R); its kernels read *n_ovf on the
// device and exit at once when the list is shorter.  Only the first chunk may
// split K (over the partial area): a later chunk runs only when more than R
// rows overflow, and without a split it launches no reduction kernels, which
// would otherwise be two more launches that exit at once in the common case.
twell_status run_fallback(const twell_matrix *m, const void *x, const void *wg, const void *wu, const void *wd,
                          const float *beta, void *y, int d, const FfnWs &L, char *base, const uint8_t *row_flag,
                          hipStream_t s) {
  const int T = m->rows, F = m->cols, R = L.chunk_rows;
  const Dt D = to_dt(m->dtype);
  TW_TRY(compact_rows(row_flag, T, m->ovf_rows, m->ovf_cap, m->n_ovf, s), "overflow row list");
  for (int c0 = 0; c0 < T; c0 += R) {
    const int rows = std::min(R, T - c0);
    const int h_cap = std::max(0, std::min(m->ovf_cap - c0, rows));
    void *h_out = (m->dense != nullptr && h_cap > 0)
                      ? static_cast<char *>(m->dense) + (size_t)c0 * F * dt_size(m->dtype)
                      : nullptr;
    DenseArgs da{D, x, wg, wu, wd, beta, y, rows, d, F, m->ovf_rows + c0, m->n_ovf, c0, base + L.a, h_out, h_cap,
                 reinterpret_cast<float *>(base + L.partial), c0 == 0 ? L.partial_tiles : 0};
    TW_TRY(dense_gate_up(da, s), "fallback gate/up matmul");
    TW_TRY(dense_down(da, s), "fallback down matmul");
  }
  return TWELL_OK;
}

twell_status run_sparse(const twell_matrix *m, const void *x, const void *wg, const void *wu, const void *wd,
                        const float *beta, void *y, int d, void *ws, const FfnWs &L, hipStream_t s) {
  const int T = m->rows, F = m->cols;
  char *base = static_cast<char *>(ws);
  uint8_t *row_flag = reinterpret_cast<uint8_t *>(base + L.flag);
  void *list = base + L.list;
  int *list_n = reinterpret_cast<int *>(base + L.list_n);
  const Dt D = to_dt(m->dtype);

  // The up kernel finds the overflow rows itself (row_flag); their list
  // follows, for the dense fallback.
  SparseArgs sa{D, T, d, F, m->tile, m->cap, m->cnt, m->val, m->idx, row_flag, x, wu, wd, list, list_n, L.stride, y,
                m->u};
  TW_TRY(sparse_up(sa, s), "sparse up projection");
  TW_TRY(sparse_down(sa, s), "sparse down projection");
  return run_fallback(m, x, wg, wu, wd, beta, y, d, L, base, row_flag, s);
}

// The hidden-group-major fused prototype: the forward's workspace followed by
// the groups' fp32 partial output rows [n_groups][T][d].
size_t grouped_partial_offset(const FfnWs &L) { return align_up(L.total, ALIGN_WS); }
size_t grouped_ws_bytes(const FfnWs &L, int T, int d, int F, int tile, twell_dtype dt) {
  const FusedGroups fg = fused_groups(d, F, tile, to_dt(dt));
  return grouped_partial_offset(L) + (size_t)fg.n_groups * T * d * 4;
}

// The same sequence with the fused up+down kernel in place of the two gather
// kernels (the compact lists are not used).
twell_status run_sparse_fused(const twell_matrix *m, const void *x, const void *wg, const void *wu, const void *wd,
                              const float *beta, void *y, int d, void *ws, const FfnWs &L, hipStream_t s,
                              bool grouped = false) {
  const int T = m->rows, F = m->cols;
  char *base = static_cast<char *>(ws);
  uint8_t *row_flag = reinterpret_cast<uint8_t *>(base + L.flag);
  const Dt D = to_dt(m->dtype);
  SparseArgs sa{D, T, d, F, m->tile, m->cap, m->cnt, m->val, m->idx, row_flag, x, wu, wd, nullptr, nullptr, 0, y,
                nullptr, m->layout == TWELL_LAYOUT_TILES};
  if (grouped) {
    TW_TRY(sparse_fused_grouped(sa, reinterpret_cast<float *>(base + grouped_partial_offset(L)), s),
           "grouped fused sparse up/down projection");
  } else {
    TW_TRY(sparse_fused(sa, s), "fused sparse up/down projection");
  }
  return run_fallback(m, x, wg, wu, wd, beta, y, d, L, base, row_flag, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of twell_ffn_forward_noalloc: the forward's workspace as a
// file-scope device array, for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy (TWELL_NOALLOC_SCRATCH_BYTES) until the
// process ends.  In host code `scratch` only names the symbol: its device
// address on the current GPU comes from hipGetSymbolAddress, taken once per
// device and kept in g_scratch_ptr, and only that address is ever passed to
// a kernel.
static __device__ __align__(256) char scratch[TWELL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// The scratch address on the current device, which must be the stream's.
twell_status scratch_address(hipStream_t s, void **out) {
  int dev = -1;
  TW_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    TW_TRY(hipStreamGetDevice(s, &sdev), "hipStreamGetDevice");
    if ((int)sdev != dev)
      return fail(TWELL_ERR_INVALID_ARG, "the stream belongs to device %d, the current device is %d", (int)sdev, dev);
  }
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(TWELL_ERR_UNSUPPORTED, "device %d: the static scratch is kept for devices 0..%d", dev,
                SCRATCH_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    TW_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(TWELL_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TWELL_OK;
}

// The forward's workspace layout within the static scratch: the default
// chunk of fallback rows, or smaller chunks (multiples of 256 rows) until it
// fits; failing that, a smaller split-K area (fewer K ranges for the
// fallback's first chunk, down to none).  false when nothing fits.
bool noalloc_layout(int T, int d, int F, int tile, int cap, twell_dtype dt, FfnWs *out) {
  for (int pcap = FALLBACK_PARTIAL_TILES_MAX;; pcap /= 2) {
    for (int R = default_chunk_rows(T); R > 0; R = R > 256 ? (R - 1) / 256 * 256 : 0) {
      const FfnWs L = ffn_ws_layout(T, d, F, tile, cap, dt, R, pcap < 2 ? 0 : pcap);
      if (L.total <= TWELL_NOALLOC_SCRATCH_BYTES) {
        *out = L;
        return true;
      }
    }
    if (pcap < 2) return false;
  }
}

}  // namespace

extern "C" {

int twell_abi_version(void) { return TWELL_ABI_VERSION; }

const char *twell_status_str(twell_status s) {
  switch (s) {
    case TWELL_OK: return "ok";
    case TWELL_ERR_INVALID_ARG: return "invalid argument";
    case TWELL_ERR_UNSUPPORTED: return "unsupported configuration";
    case TWELL_ERR_WORKSPACE: return "workspace too small";
    case TWELL_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *twell_last_error(void) { return g_err; }

twell_status twell_stream_probe(const void *src, void *dst, size_t bytes, int mode, void *stream) {
  g_err[0] = 0;
  if (mode != 0 && mode != 1) return fail(TWELL_ERR_INVALID_ARG, "mode must be 0 (read) or 1 (copy)");
  if (bytes == 0) return TWELL_OK;
  if (src == nullptr || dst == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null src or dst");
  if (bytes % 16 != 0) return fail(TWELL_ERR_UNSUPPORTED, "bytes must be a multiple of 16");
  if (!aligned(src, 16) || !aligned(dst, mode == 0 ? 4 : 16))
    return fail(TWELL_ERR_UNSUPPORTED, "misaligned probe buffer");
  return hip_check(stream_probe(src, dst, bytes, mode, static_cast<hipStream_t>(stream)), "stream probe");
}

twell_status twell_mfma_probe(float *sink, int iters, int blocks, void *stream) {
  g_err[0] = 0;
  if (sink == nullptr || iters < 1 || blocks < 1) return fail(TWELL_ERR_INVALID_ARG, "null sink, iters < 1 or blocks < 1");
  if (!aligned(sink, 4)) return fail(TWELL_ERR_UNSUPPORTED, "misaligned sink");
  return hip_check(mfma_probe(sink, iters, blocks, static_cast<hipStream_t>(stream)), "mfma probe");
}

twell_status twell_pack(const void *pre, twell_matrix *out, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(out, false);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(out, "twell_pack")) != TWELL_OK) return st;
  if ((st = check_no_u(out, "twell_pack")) != TWELL_OK) return st;
  if (out->rows > 0 && pre == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null pre");
  if (!aligned(pre, 16)) return fail(TWELL_ERR_UNSUPPORTED, "pre must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = out->rows;
  if (T == 0) return hip_check(zero_int(out->n_ovf, s), "zero n_ovf");
  const Dt D = to_dt(out->dtype);
  // With room for every row, the pack kernel writes each row's overflow flag
  // into ovf_rows and one workgroup turns the flags into the list in place;
  // otherwise a scan over the counts builds the (truncated) list.
  const bool flags_in_list = out->ovf_cap >= T;
  PackArgs pa{D, out->tile, out->cap, pre, T, out->cols, out->cnt, out->val, out->idx,
              flags_in_list ? out->ovf_rows : nullptr};
  TW_TRY(pack_tiles(pa, s), "pack");
  if (flags_in_list) {
    TW_TRY(compact_rows_in_place(out->ovf_rows, T, out->n_ovf, s), "overflow row list");
  } else {
    ScanArgs sc{out->cnt, T, out->cols / out->tile, out->cap, nullptr, out->ovf_rows, out->ovf_cap, out->n_ovf};
    TW_TRY(overflow_scan(sc, s), "overflow scan");
  }
  DenseRowsArgs dr{D, pre, T, out->cols, out->ovf_rows, out->n_ovf, out->ovf_cap, out->dense};
  TW_TRY(pack_dense_rows(dr, s), "dense rows");
  return TWELL_OK;
}

size_t twell_ffn_workspace_size(int T, int d, int F, int tile, int cap, twell_dtype dtype) {
  if (T < 0 || check_format(tile, cap, F, (int)dtype) != TWELL_OK || check_d(d, (int)dtype) != TWELL_OK ||
      check_weight_bytes(F, d, (int)dtype) != TWELL_OK)
    return 0;
  return ffn_ws_layout(T, d, F, tile, cap, dtype).total;
}

twell_status twell_gate_pack(const void *x, const void *w_gate, const float *gate_bias, int d, twell_matrix *packed,
                             void *pre_out, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, false);
  if (st != TWELL_OK) return st;
  if ((st = check_d(d, (int)packed->dtype)) != TWELL_OK) return st;
  if (packed->rows == 0) return TWELL_OK;
  if (!x || !w_gate) return fail(TWELL_ERR_INVALID_ARG, "null x/w_gate");
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(gate_bias, 4) || !aligned(pre_out, 16))
    return fail(TWELL_ERR_UNSUPPORTED, "misaligned x/w_gate/gate_bias/pre_out");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = packed->rows, F = packed->cols;
  if (T == 0) return TWELL_OK;
  GateArgs ga{to_dt(packed->dtype), packed->tile, x, w_gate, gate_bias, T, d, F, packed->cap,
              packed->cnt, packed->val, packed->idx, pre_out, packed->layout == TWELL_LAYOUT_TILES};
  TW_TRY(gate_twell(ga, s), "gate matmul");
  return TWELL_OK;
}

twell_status twell_to_hybrid(const twell_matrix *packed, twell_hybrid *out, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_to_hybrid")) != TWELL_OK) return st;
  if (out == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null twell_hybrid");
  if (out->rows != packed->rows || out->cols != packed->cols || out->dtype != packed->dtype)
    return fail(TWELL_ERR_INVALID_ARG, "hybrid rows/cols/dtype must equal the TwELL matrix's");
  if (out->width < 1) return fail(TWELL_ERR_INVALID_ARG, "width must be >= 1");
  if (out->dense_cap < 0) return fail(TWELL_ERR_INVALID_ARG, "dense_cap must be >= 0");
  if (out->n_dense == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null n_dense");
  if (out->dense_cap > 0 && out->dense_rows == nullptr)
    return fail(TWELL_ERR_INVALID_ARG, "null dense_rows with dense_cap > 0");
  const int T = packed->rows;
  if (T > 0 && (out->cnt == nullptr || out->val == nullptr || out->col == nullptr))
    return fail(TWELL_ERR_INVALID_ARG, "null cnt/val/col");
  if (T > 0 && packed->dense == nullptr)
    return fail(TWELL_ERR_INVALID_ARG, "the TwELL matrix needs its dense backup rows (packed->dense)");
  if (!aligned(out->cnt, 4) || !aligned(out->val, dt_size(out->dtype)) || !aligned(out->col, 4) ||
      !aligned(out->dense_rows, 4) || !aligned(out->n_dense, 4) || !aligned(out->dense, dt_size(out->dtype)) ||
      !aligned(out->u, 4))
    return fail(TWELL_ERR_UNSUPPORTED, "misaligned twell_hybrid buffer");
  if (out->u != nullptr && packed->u == nullptr)
    return fail(TWELL_ERR_INVALID_ARG, "out->u needs the TwELL matrix's saved u (packed->u)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return hip_check(zero_int(out->n_dense, s), "zero n_dense");
  HybridArgs ha{to_dt(packed->dtype), T, packed->cols, packed->tile, packed->cap, packed->cnt, packed->val,
                packed->idx, packed->ovf_rows, packed->n_ovf, packed->ovf_cap, packed->dense, out->width,
                out->cnt, out->val, out->col, out->dense_rows, out->n_dense, out->dense_cap, out->dense,
                out->u != nullptr ? packed->u : nullptr, out->u};
  TW_TRY(twell_to_hybrid_launch(ha, s), "TwELL to hybrid");
  return TWELL_OK;
}

size_t twell_l1_workspace_size(void) { return (size_t)L1_BLOCKS * sizeof(double); }

twell_status twell_l1_norm(const twell_matrix *packed, double *out, void *workspace, size_t ws_bytes,
                           void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_l1_norm")) != TWELL_OK) return st;
  if (out == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null out");
  if (packed->rows > 0 && packed->dense == nullptr)
    return fail(TWELL_ERR_INVALID_ARG, "the TwELL matrix needs its dense backup rows (packed->dense)");
  if (workspace == nullptr || ws_bytes < twell_l1_workspace_size())
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", twell_l1_workspace_size(),
                workspace ? ws_bytes : 0);
  if (!aligned(out, 8) || !aligned(workspace, 8)) return fail(TWELL_ERR_UNSUPPORTED, "misaligned out/workspace");
  L1Args la{to_dt(packed->dtype), packed->rows, packed->cols, packed->tile, packed->cap, packed->cnt, packed->val,
            packed->n_ovf, packed->ovf_cap, packed->dense, static_cast<double *>(workspace), out, 0.0f, nullptr,
            nullptr};
  TW_TRY(l1_norm(la, static_cast<hipStream_t>(stream)), "L1 norm");
  return TWELL_OK;
}

twell_status twell_l1_grad(const twell_matrix *packed, float lam, void *grad_val, void *grad_dense, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, false);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_l1_grad")) != TWELL_OK) return st;
  if (packed->rows > 0 && grad_val == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null grad_val");
  if (grad_dense != nullptr && packed->dense == nullptr)
    return fail(TWELL_ERR_INVALID_ARG, "grad_dense needs the TwELL matrix's dense backup rows");
  if (!aligned(grad_val, dt_size(packed->dtype)) || !aligned(grad_dense, dt_size(packed->dtype)))
    return fail(TWELL_ERR_UNSUPPORTED, "misaligned grad_val/grad_dense");
  L1Args la{to_dt(packed->dtype), packed->rows, packed->cols, packed->tile, packed->cap, packed->cnt, packed->val,
            packed->n_ovf, packed->ovf_cap, packed->dense, nullptr, nullptr, lam, grad_val, grad_dense};
  TW_TRY(l1_grad(la, static_cast<hipStream_t>(stream)), "L1 gradient");
  return TWELL_OK;
}

twell_status twell_overflow_scan(twell_matrix *packed, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, false);
  if (st != TWELL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, s), "zero n_ovf");
  ScanArgs sc{packed->cnt, packed->rows, packed->cols / packed->tile, packed->cap, nullptr, packed->ovf_rows,
              packed->ovf_cap, packed->n_ovf, packed->layout == TWELL_LAYOUT_TILES};
  TW_TRY(overflow_scan(sc, s), "overflow scan");
  return TWELL_OK;
}

twell_status twell_sparse_ffn(const twell_matrix *packed, const void *x, const void *w_gate, const void *w_up,
                              const void *w_down, const float *gate_bias, void *y, int d, void *workspace,
                              size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_sparse_ffn")) != TWELL_OK) return st;
  if ((st = check_d(d, (int)packed->dtype)) != TWELL_OK) return st;
  if ((st = check_weight_bytes(packed->cols, d, (int)packed->dtype)) != TWELL_OK) return st;
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, static_cast<hipStream_t>(stream)), "zero n_ovf");
  if ((st = check_ffn_ptrs(x, w_gate, w_up, w_down, gate_bias, y)) != TWELL_OK) return st;
  const FfnWs L = ffn_ws_layout(packed->rows, d, packed->cols, packed->tile, packed->cap, packed->dtype);
  const size_t need = L.total;
  if (workspace == nullptr || ws_bytes < need)
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (!aligned(workspace, ALIGN_WS)) return fail(TWELL_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, s), "zero n_ovf");
  return run_sparse(packed, x, w_gate, w_up, w_down, gate_bias, y, d, workspace, L, s);
}

twell_status twell_sparse_ffn_fused(const twell_matrix *packed, const void *x, const void *w_gate, const void *w_up,
                                    const void *w_down, const float *gate_bias, void *y, int d, void *workspace,
                                    size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_sparse_ffn_fused")) != TWELL_OK) return st;
  if ((st = check_no_u(packed, "twell_sparse_ffn_fused")) != TWELL_OK) return st;
  if ((st = check_d(d, (int)packed->dtype)) != TWELL_OK) return st;
  const int q = packed->dtype == TWELL_BF16 ? 512 : 256;
  if (d > 8 * q) return fail(TWELL_ERR_UNSUPPORTED, "fused kernel: d %d not built (<= %d)", d, 8 * q);
  if ((st = check_weight_bytes(packed->cols, d, (int)packed->dtype)) != TWELL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, s), "zero n_ovf");
  if ((st = check_ffn_ptrs(x, w_gate, w_up, w_down, gate_bias, y)) != TWELL_OK) return st;
  const FfnWs L = ffn_ws_layout(packed->rows, d, packed->cols, packed->tile, packed->cap, packed->dtype);
  const size_t need = L.total;
  if (workspace == nullptr || ws_bytes < need)
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (!aligned(workspace, ALIGN_WS)) return fail(TWELL_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  return run_sparse_fused(packed, x, w_gate, w_up, w_down, gate_bias, y, d, workspace, L, s);
}

size_t twell_sparse_ffn_grouped_workspace_size(int T, int d, int F, int tile, int cap, twell_dtype dtype) {
  if (T < 0 || check_format(tile, cap, F, (int)dtype) != TWELL_OK || check_d(d, (int)dtype) != TWELL_OK ||
      check_weight_bytes(F, d, (int)dtype) != TWELL_OK)
    return 0;
  return grouped_ws_bytes(ffn_ws_layout(T, d, F, tile, cap, dtype), T, d, F, tile, dtype);
}

twell_status twell_sparse_ffn_grouped(const twell_matrix *packed, const void *x, const void *w_gate,
                                      const void *w_up, const void *w_down, const float *gate_bias, void *y, int d,
                                      void *workspace, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_no_u(packed, "twell_sparse_ffn_grouped")) != TWELL_OK) return st;
  if ((st = check_d(d, (int)packed->dtype)) != TWELL_OK) return st;
  const int q = packed->dtype == TWELL_BF16 ? 512 : 256;
  if (d > 8 * q) return fail(TWELL_ERR_UNSUPPORTED, "grouped fused kernel: d %d not built (<= %d)", d, 8 * q);
  if ((st = check_weight_bytes(packed->cols, d, (int)packed->dtype)) != TWELL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, s), "zero n_ovf");
  if ((st = check_ffn_ptrs(x, w_gate, w_up, w_down, gate_bias, y)) != TWELL_OK) return st;
  const FfnWs L = ffn_ws_layout(packed->rows, d, packed->cols, packed->tile, packed->cap, packed->dtype);
  const size_t need = grouped_ws_bytes(L, packed->rows, d, packed->cols, packed->tile, packed->dtype);
  if (workspace == nullptr || ws_bytes < need)
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (!aligned(workspace, ALIGN_WS)) return fail(TWELL_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  return run_sparse_fused(packed, x, w_gate, w_up, w_down, gate_bias, y, d, workspace, L, s, true);
}

twell_status twell_ffn_forward(const void *x, const void *w_gate, const void *w_up, const void *w_down,
                               const float *gate_bias, void *y, int d, twell_matrix *packed, void *workspace,
                               size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_ffn_forward")) != TWELL_OK) return st;
  if ((st = check_d(d, (int)packed->dtype)) != TWELL_OK) return st;
  if ((st = check_weight_bytes(packed->cols, d, (int)packed->dtype)) != TWELL_OK) return st;
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, static_cast<hipStream_t>(stream)), "zero n_ovf");
  if ((st = check_ffn_ptrs(x, w_gate, w_up, w_down, gate_bias, y)) != TWELL_OK) return st;
  const FfnWs L = ffn_ws_layout(packed->rows, d, packed->cols, packed->tile, packed->cap, packed->dtype);
  const size_t need = L.total;
  if (workspace == nullptr || ws_bytes < need)
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (!aligned(workspace, ALIGN_WS)) return fail(TWELL_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = packed->rows, F = packed->cols;
  if (T == 0) return hip_check(zero_int(packed->n_ovf, s), "zero n_ovf");
  GateArgs ga{to_dt(packed->dtype), packed->tile, x, w_gate, gate_bias, T, d, F, packed->cap,
              packed->cnt, packed->val, packed->idx, nullptr};
  TW_TRY(gate_twell(ga, s), "gate matmul");
  return run_sparse(packed, x, w_gate, w_up, w_down, gate_bias, y, d, workspace, L, s);
}

twell_status twell_ffn_forward_noalloc(const void *x, const void *w_gate, const void *w_up, const void *w_down,
                                       const float *gate_bias, void *y, int d, twell_matrix *packed, void *stream) {
  g_err[0] = 0;
  twell_status st = check_matrix(packed, true);
  if (st != TWELL_OK) return st;
  if ((st = check_rows_layout(packed, "twell_ffn_forward_noalloc")) != TWELL_OK) return st;
  if ((st = check_d(d, (int)packed->dtype)) != TWELL_OK) return st;
  if ((st = check_weight_bytes(packed->cols, d, (int)packed->dtype)) != TWELL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (packed->rows == 0) return hip_check(zero_int(packed->n_ovf, s), "zero n_ovf");
  if ((st = check_ffn_ptrs(x, w_gate, w_up, w_down, gate_bias, y)) != TWELL_OK) return st;
  const int T = packed->rows, F = packed->cols;
  FfnWs L;
  if (!noalloc_layout(T, d, F, packed->tile, packed->cap, packed->dtype, &L))
    return fail(TWELL_ERR_WORKSPACE,
                "the forward of T=%d, d=%d, F=%d needs %zu bytes of workspace even with 256-row fallback chunks "
                "and no split-K area; the static scratch holds %zu",
                T, d, F, ffn_ws_layout(T, d, F, packed->tile, packed->cap, packed->dtype, std::min(T, 256), 0).total,
                (size_t)TWELL_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((st = scratch_address(s, &ws)) != TWELL_OK) return st;
  GateArgs ga{to_dt(packed->dtype), packed->tile, x, w_gate, gate_bias, T, d, F, packed->cap,
              packed->cnt, packed->val, packed->idx, nullptr};
  TW_TRY(gate_twell(ga, s), "gate matmul");
  return run_sparse(packed, x, w_gate, w_up, w_down, gate_bias, y, d, ws, L, s);
}

}  // extern "C"

namespace {

// The backward's gather kernels hold x_t and dy_t in registers (at most 8
// 16-byte chunks per lane each) and cut d into 128-column slices; its
// transpose keeps a 64-bit mask per hidden unit in LDS.
constexpr int BW_MAX_F = 16384;

twell_status check_backward_shape(int T, int d, int F, int width, int dense_cap, int dtype) {
  if (!valid_dtype(dtype)) return fail(TWELL_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (T < 0 || F <= 0 || width < 1 || dense_cap < 0)
    return fail(TWELL_ERR_INVALID_ARG, "need rows >= 0, cols > 0, width >= 1, dense_cap >= 0");
  if (d <= 0) return fail(TWELL_ERR_INVALID_ARG, "d must be positive");
  const int q = dtype == TWELL_BF16 ? 512 : 256;
  if (d % q != 0 || d > 8 * q)
    return fail(TWELL_ERR_UNSUPPORTED, "backward: d %d not built (multiple of %d, <= %d)", d, q, 8 * q);
  if (F > BW_MAX_F) return fail(TWELL_ERR_UNSUPPORTED, "backward: cols %d not built (<= %d)", F, BW_MAX_F);
  twell_status st = check_weight_bytes(F, d, dtype);
  if (st != TWELL_OK) return st;
  if ((size_t)T * d * dt_size((twell_dtype)dtype) >= ((size_t)1 << 31))
    return fail(TWELL_ERR_UNSUPPORTED, "backward: x / dy of T*d = %zu elements are too large", (size_t)T * d);
  if ((size_t)T * width + (size_t)dense_cap * F >= ((size_t)1 << 31))
    return fail(TWELL_ERR_UNSUPPORTED, "backward: rows*width + dense_cap*cols must stay below 2^31 entries");
  return TWELL_OK;
}

// The dense backup rows go to the matrix-core kernels when the hidden size is
// a multiple of their 128-unit tiles; otherwise their entries are walked like
// the others.
bool bw_dense_mma(int F) { return F % 128 == 0; }

// Workspace of the backward: compacted dense rows | per-entry (du, dpre) |
// per-entry column-major position | column-major records | per-block column
// counts | their running offsets | column totals | column starts | row order,
// then the matrix-core dense-row pieces: gathered x and dy rows | du and dpre
// rows | a, du, dpre transposed | the dx split's partial tiles.  The dense
// rows' entry slots and compacted columns exist only without the matrix-core
// path.
struct BwWs {
  size_t dcol, dn, ent, pos, csc, blk, boff, tot, colptr, order;
  size_t xr, dyr, du, dp, at, dut, dpt, part;
  int part_tiles, as_stride;
  size_t total;
};

BwWs bw_ws_layout(int T, int d, int F, int width, int dense_cap, twell_dtype dtype) {
  BwWs w;
  const bool mma = bw_dense_mma(F);
  const size_t NE = (size_t)T * width + (mma ? 0 : (size_t)dense_cap * F);
  const size_t NB = ((size_t)T + 63) / 64;
  const size_t dcap_lists = mma ? 0 : (size_t)dense_cap;
  w.dcol = 0;
  w.dn = align_up(w.dcol + dcap_lists * F * 4, ALIGN_WS);
  w.ent = align_up(w.dn + dcap_lists * 4, ALIGN_WS);
  w.pos = align_up(w.ent + NE * 8, ALIGN_WS);
  w.csc = align_up(w.pos + NE * 4, ALIGN_WS);
  w.blk = align_up(w.csc + NE * 16, ALIGN_WS);
  w.boff = align_up(w.blk + NB * F, ALIGN_WS);
  w.tot = align_up(w.boff + NB * F * 4, ALIGN_WS);
  w.colptr = align_up(w.tot + (size_t)F * 4, ALIGN_WS);
  w.order = align_up(w.colptr + ((size_t)F + 1) * 4, ALIGN_WS);
  size_t end = align_up(w.order + (size_t)T * 4, ALIGN_WS);
  const size_t s = dt_size(dtype);
  const bool dense = mma && dense_cap > 0 && T > 0;
  const int ns = dtype == TWELL_BF16 ? 2 : 1;
  w.as_stride = dense ? ns * twell::backward_dense_rows_padded(dense_cap, to_dt(dtype)) : 0;
  w.part_tiles = dense ? twell::backward_dense_partial_tiles(dense_cap, d) : 0;
  const size_t g = dense ? (size_t)w.as_stride * d * s : 0;            // gathered rows
  const size_t rm = dense ? (size_t)dense_cap * F * s : 0;             // du / dpre rows
  const size_t tr = dense ? (size_t)F * w.as_stride * s : 0;           // transposed operands
  w.xr = end;
  w.dyr = align_up(w.xr + g, ALIGN_WS);
  w.du = align_up(w.dyr + g, ALIGN_WS);
  w.dp = align_up(w.du + rm, ALIGN_WS);
  w.at = align_up(w.dp + rm, ALIGN_WS);
  w.dut = align_up(w.at + tr, ALIGN_WS);
  w.dpt = align_up(w.dut + tr, ALIGN_WS);
  w.part = align_up(w.dpt + tr, ALIGN_WS);
  w.total = align_up(w.part + (size_t)w.part_tiles * twell::FALLBACK_SPLIT_TILE * 4, ALIGN_WS);
  return w;
}

}  // namespace

extern "C" {

size_t twell_ffn_backward_workspace_size(int T, int d, int F, int width, int dense_cap, twell_dtype dtype) {
  char saved[sizeof(g_err)];
  memcpy(saved, g_err, sizeof(g_err));
  const twell_status st = check_backward_shape(T, d, F, width, dense_cap, (int)dtype);
  memcpy(g_err, saved, sizeof(g_err));
  if (st != TWELL_OK) return 0;
  return bw_ws_layout(T, d, F, width, dense_cap, dtype).total;
}

twell_status twell_ffn_backward(const twell_hybrid *h, const void *x, const void *w_gate, const void *w_up,
                                const void *w_down, const void *dy, float lam, int d, void *dx, float *dw_gate,
                                float *dw_up, float *dw_down, void *workspace, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (h == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null twell_hybrid");
  twell_status st = check_backward_shape(h->rows, d, h->cols, h->width, h->dense_cap, (int)h->dtype);
  if (st != TWELL_OK) return st;
  const int T = h->rows, F = h->cols;
  if (h->n_dense == nullptr) return fail(TWELL_ERR_INVALID_ARG, "null n_dense");
  if (T > 0 && (h->cnt == nullptr || h->val == nullptr || h->col == nullptr))
    return fail(TWELL_ERR_INVALID_ARG, "null cnt/val/col");
  if (h->dense_cap > 0 && (h->dense_rows == nullptr || h->dense == nullptr))
    return fail(TWELL_ERR_INVALID_ARG, "dense_cap > 0 needs dense_rows and the dense backup rows");
  if (!aligned(h->cnt, 4) || !aligned(h->val, dt_size(h->dtype)) || !aligned(h->col, 4) ||
      !aligned(h->dense_rows, 4) || !aligned(h->n_dense, 4) || !aligned(h->dense, dt_size(h->dtype)) ||
      !aligned(h->u, 4))
    return fail(TWELL_ERR_UNSUPPORTED, "misaligned twell_hybrid buffer");
  if (!w_gate || !w_up || !w_down || !dw_gate || !dw_up || !dw_down)
    return fail(TWELL_ERR_INVALID_ARG, "null weight or weight-gradient pointer");
  if (T > 0 && (!x || !dy || !dx)) return fail(TWELL_ERR_INVALID_ARG, "null x/dy/dx");
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) ||
      !aligned(w_down, 16) || !aligned(dw_gate, 16) || !aligned(dw_up, 16) || !aligned(dw_down, 16))
    return fail(TWELL_ERR_UNSUPPORTED, "x, dy, dx, weights and weight gradients must be 16-byte aligned");
  if (h->dense_cap > 0 && bw_dense_mma(F) && !aligned(h->dense, 16))
    return fail(TWELL_ERR_UNSUPPORTED, "the dense backup rows must be 16-byte aligned");
  const BwWs L = bw_ws_layout(T, d, F, h->width, h->dense_cap, h->dtype);
  if (workspace == nullptr || ws_bytes < L.total)
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace ? ws_bytes : 0);
  if (!aligned(workspace, ALIGN_WS)) return fail(TWELL_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  char *base = static_cast<char *>(workspace);
  BackwardArgs ba{to_dt(h->dtype), T, d, F, h->width, h->cnt, h->val, h->col, h->dense_rows, h->n_dense,
                  h->dense_cap, h->dense, x, dy, w_gate, w_up, w_down, lam, dx, dw_gate, dw_up, dw_down,
                  reinterpret_cast<int *>(base + L.dcol), reinterpret_cast<int *>(base + L.dn), base + L.ent,
                  reinterpret_cast<int *>(base + L.pos), base + L.csc, reinterpret_cast<uint8_t *>(base + L.blk),
                  reinterpret_cast<int *>(base + L.boff), reinterpret_cast<int *>(base + L.tot),
                  reinterpret_cast<int *>(base + L.colptr), reinterpret_cast<int *>(base + L.order),
                  bw_dense_mma(F), base + L.xr, base + L.dyr, base + L.du, base + L.dp, base + L.at,
                  base + L.dut, base + L.dpt, reinterpret_cast<float *>(base + L.part), L.part_tiles, h->u};
  TW_TRY(ffn_backward(ba, static_cast<hipStream_t>(stream)), "FFN backward");
  return TWELL_OK;
}

size_t dense_ffn_workspace_size(int T, int d, int F, twell_dtype dtype) {
  if (T < 0 || !valid_dtype((int)dtype) || F <= 0 || F % 128 != 0 || F > (1 << 24) ||
      check_d(d, (int)dtype) != TWELL_OK)
    return 0;
  return std::max(align_up((size_t)T * F * dt_size(dtype), ALIGN_WS), ALIGN_WS);
}

twell_status dense_ffn_forward(const void *x, const void *w_gate, const void *w_up, const void *w_down,
                               const float *gate_bias, void *y, int T, int d, int F, twell_dtype dtype,
                               void *workspace, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (!valid_dtype((int)dtype)) return fail(TWELL_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (T < 0 || F <= 0) return fail(TWELL_ERR_INVALID_ARG, "T must be >= 0 and F > 0");
  if (F % 128 != 0 || F > (1 << 24)) return fail(TWELL_ERR_UNSUPPORTED, "F %d not built (multiple of 128)", F);
  twell_status st = check_d(d, (int)dtype);
  if (st != TWELL_OK) return st;
  if ((st = check_weight_bytes(F, d, (int)dtype)) != TWELL_OK) return st;
  if (T == 0) return TWELL_OK;
  if ((st = check_ffn_ptrs(x, w_gate, w_up, w_down, gate_bias, y)) != TWELL_OK) return st;
  const size_t need = dense_ffn_workspace_size(T, d, F, dtype);
  if (workspace == nullptr || ws_bytes < need)
    return fail(TWELL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (!aligned(workspace, ALIGN_WS)) return fail(TWELL_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (T == 0) return TWELL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DenseArgs da{to_dt(dtype), x, w_gate, w_up, w_down, gate_bias, y, T, d, F, nullptr, nullptr, 0, workspace,
               nullptr, 0, nullptr, 0};
  TW_TRY(dense_gate_up(da, s), "dense gate/up matmul");
  TW_TRY(dense_down(da, s), "dense down matmul");
  return TWELL_OK;
}

}  // extern "C"
