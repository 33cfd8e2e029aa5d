/*
 * twell.h -- C ABI of the MI355X (gfx950) TwELL sparse-FFN library (libtwell.so).
 *
 * The library computes the forward pass of one ReLU-gated ("ReGLU")
 * transformer feed-forward layer
 *
 *     pre = x W_g^T + beta,   h = ReLU(pre),   u = x W_u^T,   y = (h * u) W_d
 *
 * where the gate activations h are about 99% zero and are carried in the
 * TwELL (tile-wise ELLPACK) format, with a dense backup for rows that do not
 * fit.  Sources: gist.science "Sparser, Faster, Lighter Transformer Language
 * Models", Resumen Técnico §2.A (TwELL: hidden columns cut into tiles, the
 * non-zeros of each tile packed in the epilogue of the dense gate matmul, no
 * separate conversion pass; hybrid format with a dense backup matrix for
 * overflowing rows) and §2.B (inference kernel: up and down projections driven
 * by the TwELL gate activations); q2bstudio post on TwELL, third and fourth
 * paragraphs (ReLU in place of SiLU; compact ELL plus dense backup for rows
 * with many non-zeros); estadored.mx news item on the same paper (TwELL cuts
 * index management and memory traffic).  The pages fix no layout, precision
 * or tile size; every such choice below is this library's own definition.
 *
 * General rules for every entry point
 * -----------------------------------
 * - Pointers inside arguments are DEVICE pointers unless stated otherwise.
 *   Structures passed by pointer (twell_matrix) live in HOST memory.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL = the default stream).  The library never allocates device memory,
 *   never synchronises the host and keeps no pointer after returning.
 * - Arguments are validated on the host before any HIP call.  On any error
 *   status nothing has been launched and every output is untouched.
 * - Device buffers must be 16-byte aligned (torch allocations are).
 * - Dtypes: TWELL_F32 (IEEE binary32) or TWELL_BF16 (bfloat16, bit pattern
 *   in a uint16).  All dot products accumulate in fp32; stored values are
 *   rounded to the storage dtype with round-to-nearest-even.
 * - Shapes: T tokens (T >= 0; T == 0 is a no-op apart from *n_ovf = 0, and
 *   x and y may then be NULL),
 *   d = d_model, F = d_ff.  d must be a multiple of 256 and at most 4096
 *   (fp32), or a multiple of 512 and at most 8192 (bf16); F must be a
 *   multiple of the TwELL tile width, and one weight matrix (F*d elements)
 *   must stay below 2 GiB.
 * - Weights are rows per hidden unit, row-major: w_gate [F][d] (= W_g^T, the
 *   nn.Linear weight layout), w_up [F][d] (= W_u^T), w_down [F][d] (= W_d,
 *   transposed once at load time so that every hidden unit's down row is
 *   contiguous).  x and y are [T][d] row-major.  gate_bias is one fp32 value
 *   per token ([T]) or NULL for none.
 * - Inactive units contribute nothing (the pages' exactness argument for
 *   skipping zeros, gist.science Resumen Técnico §2.B): on the sparse path a
 *   token's output depends only on the w_up and w_down rows of its active
 *   units, so a non-finite weight in the row of a unit that is inactive for
 *   that token does not reach it.  Rows that take the dense fallback (and
 *   dense_ffn_forward) go through dense matmuls, where such a weight gives
 *   0 * inf = NaN as in any dense product: there weights must be finite.
 * - Thread safety: every entry point is reentrant; calls on different
 *   streams do not interact.  twell_last_error() is thread-local.
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TWELL_ABI_VERSION 3

/* The enums are int-sized.  Compiled as C++ they have the fixed underlying
 * type int, so any int a C caller stores in one is a value of the type, which
 * the library then validates (an unknown dtype is TWELL_ERR_INVALID_ARG, an
 * unknown status has the string "unknown status"). */
#ifdef __cplusplus
#define TWELL_ENUM_BASE : int
#else
#define TWELL_ENUM_BASE
#endif

typedef enum TWELL_ENUM_BASE {
  TWELL_OK = 0,
  TWELL_ERR_INVALID_ARG = 1, /* NULL required pointer, bad enum, negative or inconsistent size */
  TWELL_ERR_UNSUPPORTED = 2, /* valid but not built: tile, cap, d, dtype or alignment */
  TWELL_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the *_workspace_size() value */
  TWELL_ERR_HIP = 4          /* a HIP call or kernel launch failed; see twell_last_error() */
} twell_status;

typedef enum TWELL_ENUM_BASE { TWELL_F32 = 0, TWELL_BF16 = 1 } twell_dtype;

/* Order of the (row, tile) records of a TwELL matrix (see twell_matrix). */
typedef enum TWELL_ENUM_BASE { TWELL_LAYOUT_ROWS = 0, TWELL_LAYOUT_TILES = 1 } twell_layout;

/*
 * One TwELL matrix [rows][cols] (token-major), described by caller-owned
 * device buffers.  Definition (this library's reading of the TwELL format,
 * gist.science Resumen Técnico §2.A):
 *
 *   A value v is ACTIVE iff IEEE v > 0, decided on the stored bits: fp32
 *   0 < bits <= 0x7F800000, bf16 0 < bits <= 0x7F80 (bits read as signed).
 *   +denormals and +inf are active; +-0, negatives and NaNs are not.
 *
 *   For row t and tile k (columns [k*tile, (k+1)*tile)):
 *     cnt[t][k]          number of active columns in the tile (NOT capped).
 *     val[t][k][s],      for s < min(cnt, cap): the bits of the s-th active
 *     idx[t][k][s]       column in ascending column order, and its offset
 *                        inside the tile (0..tile-1).  Slots s >= cnt hold
 *                        +0 and 0.  A consumer takes an index modulo the
 *                        tile width, so a malformed index (>= tile) can
 *                        only name a column of its own tile.
 *   Row t OVERFLOWS iff cnt[t][k] > cap for some k (cnt == cap still fits).
 *   Its TwELL slots still hold the first min(cnt, cap) entries per tile.
 *     ovf_rows[r]        the overflowing rows in ascending order, r < n_ovf.
 *     *n_ovf             the true number of overflowing rows (may exceed
 *                        ovf_cap, in which case only ovf_cap are listed).
 *     dense[r][:]        ReLU of overflow row ovf_rows[r] (active values bit
 *                        for bit, +0 elsewhere), r < min(n_ovf, ovf_cap);
 *                        the dense backup of the hybrid format.
 *     u[t][k][s]         optional (NULL: none): for a row that did not
 *                        overflow, the up-projection value x_t . W_u[j] (fp32)
 *                        of the unit j of each used slot, saved by the forward
 *                        (twell_ffn_forward, twell_ffn_forward_noalloc,
 *                        twell_sparse_ffn) so that the backward need not
 *                        recompute it; every slot of an overflow row holds
 *                        NaN (not saved).  Slots past the count are not
 *                        written.  The other producers of a TwELL matrix
 *                        (twell_pack) and the fused prototypes take u == NULL.
 *
 *   Layout.  The record of (row t, tile k) -- its count and its cap slots --
 *   sits at position r = t * (cols/tile) + k (TWELL_LAYOUT_ROWS, the default:
 *   a row's records are contiguous) or r = k * rows + t (TWELL_LAYOUT_TILES:
 *   a tile's records are contiguous, for consumers that walk the hidden units
 *   tile by tile over all tokens): cnt[r], val[r][s], idx[r][s], u[r][s].
 *   The tile-major layout is written by twell_gate_pack and read by
 *   twell_overflow_scan and twell_sparse_ffn_grouped (the hidden-group-major
 *   fused prototype, gist.science Resumen Técnico §2.B); it carries no u.
 *   Every other entry point takes TWELL_LAYOUT_ROWS only and returns
 *   TWELL_ERR_UNSUPPORTED for the other.
 */
typedef struct {
  int32_t rows, cols;   /* T, F; cols % tile == 0 */
  int32_t tile;         /* W: 128 or 256 */
  int32_t cap;          /* C: 1 <= cap <= min(tile, 64) */
  twell_dtype dtype;    /* value dtype == activation dtype */
  uint16_t *cnt;        /* [rows][cols/tile] ([cols/tile][rows] tile-major) */
  void *val;            /* [rows][cols/tile][cap], dtype (tile-major: [cols/tile][rows][cap]) */
  uint8_t *idx;         /* [rows][cols/tile][cap] (tile-major: [cols/tile][rows][cap]) */
  int32_t *ovf_rows;    /* [ovf_cap] */
  int32_t *n_ovf;       /* [1] */
  void *dense;          /* [ovf_cap][cols], dtype; may be NULL (not written) */
  int32_t ovf_cap;      /* rows available in ovf_rows (and dense when non-NULL) */
  float *u;             /* [rows][cols/tile][cap] fp32, or NULL (see above) */
  twell_layout layout;  /* record order (see above); TWELL_LAYOUT_ROWS unless stated */
} twell_matrix;

/* ABI version of the loaded library (TWELL_ABI_VERSION). */
int twell_abi_version(void);

/* Static text for a status code. */
const char *twell_status_str(twell_status s);

/* Text of the last TWELL_ERR_HIP (or validation) error on this thread; "" if none. */
const char *twell_last_error(void);

/*
 * twell_pack -- pack a given pre-activation tensor into TwELL.
 *
 * pre: [out->rows][out->cols] device buffer in out->dtype.  Fills every field
 * of *out as defined above: cnt, val, idx, ovf_rows (first ovf_cap),
 * *n_ovf, and dense (when non-NULL).  Entries of ovf_rows at and past
 * min(n_ovf, ovf_cap) are unspecified on return: when ovf_cap >= rows the
 * call keeps one overflow flag per row there before listing the rows.  This is the format of gist.science
 * Resumen Técnico §2.A applied to an explicit matrix; twell_ffn_forward
 * produces the same TwELL matrix inside the gate matmul.
 * Errors: INVALID_ARG (NULL pre/out/cnt/val/idx/n_ovf, ovf_rows NULL with
 * ovf_cap > 0, rows < 0, ovf_cap < 0, cols <= 0, cols % tile != 0),
 * UNSUPPORTED (tile, cap, dtype, alignment), HIP.
 */
twell_status twell_pack(const void *pre, twell_matrix *out, void *stream);

/*
 * Workspace bytes needed by twell_ffn_forward / twell_sparse_ffn /
 * twell_sparse_ffn_fused for the given shape and format (0 on invalid
 * arguments).  The layout (each piece 256-byte aligned): one flag byte and one
 * int32 entry count per row; a region shared by the per-row entry lists
 * (F/tile*cap pairs of (weight-row offset, v) per row, 8 bytes each, rounded
 * up to 8 pairs) and, once the down projection has consumed them, the dense
 * fallback's activations for one chunk of R overflow rows ([R][F] in the
 * storage dtype, R = T for T <= 512, else ceil(T/2) rounded up to 256); and
 * the fp32 partial tiles of the fallback's split-K (256 x 256 floats each, at
 * most 128, only as many as a split can use for chunks of R rows).  At
 * T = 8192, d = 2048, F = 8192, tile 256, cap 16, bf16 this is 96 MiB, below
 * the 128 MiB of the dense activation matrix the format replaces.
 */
size_t twell_ffn_workspace_size(int T, int d, int F, int tile, int cap, twell_dtype dtype);

/*
 * twell_ffn_forward -- the sparse ReGLU FFN forward:
 *   y = (ReLU(x W_g^T + beta) * (x W_u^T)) W_d
 * computed as (1) the dense gate matmul on the matrix cores whose epilogue
 * adds beta, rounds to the storage dtype, applies ReLU and writes TwELL into
 * *packed directly (no dense pre-activation matrix is stored); (2) the
 * overflow test of every row (some tile counts more than cap entries) and the
 * ascending list of the overflowing rows; (3) the up projection for the
 * active entries of non-overflowing rows only; (4) the down projection as a
 * weighted sum of w_down rows, fp32 accumulation, one rounding to the storage
 * dtype; (5) the dense fallback (gate, up and down matmuls) for the
 * overflowing rows, which also writes packed->dense when it is non-NULL.
 * Step (2) runs inside the up projection's kernel, which reads every row's
 * counts anyway, plus a one-pass compaction of the row flags.
 * Sources: gist.science Resumen Técnico §2.A and §2.B.
 *
 * packed: caller-owned TwELL buffers with rows == T, cols == F; tile, cap and
 * dtype select the format and the arithmetic.  packed->ovf_cap must be >= T so
 * that no overflowing row can be dropped.  On return (after the stream
 * completes) *packed describes round(pre) exactly as twell_pack would.  With
 * packed->u non-NULL the up projection also saves u = x_t . W_u[j] (fp32) of
 * every used slot of a non-overflow row, and NaN in every slot of an
 * overflow row (the training forward: the backward then skips one gather).
 * y: [T][d] in the storage dtype, fully written.
 * workspace: device buffer of at least twell_ffn_workspace_size() bytes,
 * 256-byte aligned; its contents on entry do not matter (layout above).  The
 * fallback runs over the overflow list in chunks of R rows, so any number of
 * overflowing rows, up to all T, is computed; when they are too few to fill
 * the GPU the first chunk splits K into ranges whose fp32 partial tiles are
 * added in a fixed order, so y stays deterministic.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
twell_status twell_ffn_forward(const void *x, const void *w_gate, const void *w_up,
                               const void *w_down, const float *gate_bias, void *y, int d,
                               twell_matrix *packed, void *workspace, size_t ws_bytes,
                               void *stream);

/*
 * twell_ffn_forward_noalloc -- twell_ffn_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, kernels and results,
 * with the workspace taken from a static device array of
 * TWELL_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates nothing.  The fallback's row
 * chunk is the largest (multiple of 256 rows, at most the default) whose
 * workspace fits; shapes whose workspace does not fit even with 256-row
 * chunks are rejected with TWELL_ERR_WORKSPACE before any launch (the
 * 1.5B-class layer, T = 8192, d = 2048, F = 8192, bf16, fits).
 * The stream must belong to the current device.  Every call on one GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (different
 * streams, or different host threads) race and must be serialised by the
 * caller.  The array's contents between calls do not matter.
 * Errors: as twell_ffn_forward, WORKSPACE when the shape needs more than the
 * static scratch, INVALID_ARG when the stream is another device's.
 */
#define TWELL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
twell_status twell_ffn_forward_noalloc(const void *x, const void *w_gate, const void *w_up,
                                       const void *w_down, const float *gate_bias, void *y, int d,
                                       twell_matrix *packed, void *stream);

/*
 * Stage entry points (for profiling and parity).  twell_ffn_forward performs
 * twell_gate_pack followed by twell_sparse_ffn on the same arguments.
 *
 * twell_gate_pack: step (1) alone -- one kernel, the gate matmul with the
 * TwELL epilogue: the dense matmul whose epilogue materialises the sparse
 * activations in TwELL with no separate conversion pass and no
 * synchronisation between thread blocks (gist.science Resumen Técnico §2.A;
 * the estadored.mx item on the same paper, on the index management and
 * memory traffic this avoids).  Writes packed->cnt, val and idx; ovf_rows, n_ovf and dense
 * are not touched (twell_overflow_scan completes them).  With
 * packed->layout == TWELL_LAYOUT_TILES the records are written tile-major
 * (the same values at the other record positions).  pre_out, when
 * non-NULL, receives the rounded pre-activations [T][F] in the storage dtype
 * (a debugging dump; the fused path itself never stores them).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
twell_status twell_gate_pack(const void *x, const void *w_gate, const float *gate_bias, int d,
                             twell_matrix *packed, void *pre_out, void *stream);

/*
 * twell_overflow_scan: step (2) alone.  Reads packed->cnt (either layout)
 * and writes the ascending list of overflowing rows (first ovf_cap of them)
 * and *n_ovf.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
twell_status twell_overflow_scan(twell_matrix *packed, void *stream);

/*
 * twell_sparse_ffn: steps (2)-(5) from the cnt/val/idx written by
 * twell_gate_pack (or by twell_pack of the rounded gate pre-activations): the
 * inference route of gist.science Resumen Técnico §2.B (up and down
 * projections over the active gate units only) plus the dense backup for
 * rows with many non-zeros (§2.A; q2bstudio post on TwELL, third paragraph).  It
 * rebuilds the overflow list itself; the overflow rows' gate is recomputed from
 * x, w_gate and gate_bias, and packed->dense is written when non-NULL.
 */
twell_status twell_sparse_ffn(const twell_matrix *packed, const void *x, const void *w_gate,
                              const void *w_up, const void *w_down, const float *gate_bias,
                              void *y, int d, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes needed by dense_ffn_forward (0 on invalid arguments). */
size_t dense_ffn_workspace_size(int T, int d, int F, twell_dtype dtype);

/*
 * dense_ffn_forward -- the same layer computed densely on the matrix cores
 * (the baseline the sparse path is measured against: GPUs are built for
 * dense products and sparse kernels used to lose to them, gist.science
 * Resumen Técnico §1 and the q2bstudio post's first paragraph; the forward
 * speedups of §4 are over dense execution): a fused gate+up matmul
 * whose epilogue forms a = ReLU(round(pre)) * u rounded to the storage dtype,
 * then the down matmul y = a W_d.  Same argument conventions as
 * twell_ffn_forward.  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
twell_status dense_ffn_forward(const void *x, const void *w_gate, const void *w_up,
                               const void *w_down, const float *gate_bias, void *y, int T,
                               int d, int F, twell_dtype dtype, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * twell_hybrid -- the hybrid format for training activations: rows with few
 * non-zeros as rows of a compact ELL matrix, rows with many in a dense backup
 * matrix (gist.science "Sparser, Faster, Lighter Transformer Language Models",
 * Resumen Técnico §2.A; q2bstudio post on TwELL, third paragraph).  The pages
 * fix no width or layout; here, for a row t of the activation matrix:
 *     cnt[t]             number of active entries (IEEE v > 0 on the bits).
 *     ELL row            iff cnt[t] <= width: val[t][s], col[t][s] for
 *                        s < cnt[t] hold the s-th active entry in ascending
 *                        column order (value bits, column index); every other
 *                        slot holds +0 and column 0.
 *     dense row          iff cnt[t] > width: its ELL slots are all padding,
 *                        t is listed in dense_rows (ascending; *n_dense is the
 *                        true count, only the first dense_cap are listed) and
 *                        dense[r][:] holds ReLU(row dense_rows[r]) when dense
 *                        is non-NULL.
 *     u[t][s]            optional (NULL: none): for an ELL row, the saved
 *                        up-projection value of slot s < cnt[t] (fp32), from
 *                        the TwELL matrix's u; NaN in u[t][0] marks a row whose
 *                        u was not saved (its TwELL row overflowed).  Other
 *                        slots are not written.
 */
typedef struct {
  int32_t rows, cols;    /* T, F: as the TwELL matrix converted */
  int32_t width;         /* ELL slots per row, >= 1 */
  twell_dtype dtype;     /* value dtype */
  int32_t *cnt;          /* [rows] */
  void *val;             /* [rows][width], dtype */
  int32_t *col;          /* [rows][width] */
  int32_t *dense_rows;   /* [dense_cap] */
  int32_t *n_dense;      /* [1] */
  void *dense;           /* [dense_cap][cols], dtype; may be NULL (not written) */
  int32_t dense_cap;     /* rows available in dense_rows (and dense) */
  float *u;              /* [rows][width] fp32, or NULL (see above) */
} twell_hybrid;

/*
 * twell_to_hybrid -- convert a TwELL matrix to the hybrid format (the training
 * conversion kernel of the same summary, §2.B).  The result is the hybrid of
 * the activation matrix the TwELL matrix describes, whatever its tile and
 * capacity: rows that overflowed TwELL are taken from packed->dense, so
 * packed->dense must be non-NULL and packed->ovf_cap >= packed->rows (as
 * written by twell_pack, or by twell_ffn_forward with a dense buffer).
 * out: caller-owned buffers with rows, cols and dtype equal to packed's.
 * out->u non-NULL: the saved u of the ELL rows is copied from packed->u, which
 * must then be non-NULL.
 * Errors: INVALID_ARG, UNSUPPORTED (alignment), HIP.
 */
twell_status twell_to_hybrid(const twell_matrix *packed, twell_hybrid *out, void *stream);

/*
 * The L1 activation penalty of the training recipe (gist.science "Sparser,
 * Faster, Lighter Transformer Language Models", Resumen Técnico §2.B,
 * training-strategy paragraph; §4: coefficient 2e-5), from TwELL without
 * expanding the activations.  The pages do not fix the normalisation: the
 * penalty is lam * ||h||_1 over all entries of h = ReLU(pre), any per-token
 * or per-unit scaling folded into lam by the caller.
 *
 * twell_l1_norm: *out (device double) = ||h||_1, float64 sums in a fixed
 * order (deterministic).  Reads the used slots of rows that did not overflow
 * and the dense backup rows of those that did, so packed->dense must be
 * non-NULL and packed->ovf_cap >= packed->rows.  workspace: device buffer of
 * at least twell_l1_workspace_size() bytes, 8-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED (alignment), WORKSPACE, HIP.
 */
size_t twell_l1_workspace_size(void);
twell_status twell_l1_norm(const twell_matrix *packed, double *out, void *workspace, size_t ws_bytes,
                           void *stream);

/*
 * twell_l1_grad: d(lam ||h||_1)/dh in the TwELL matrix's own pattern (the
 * subgradient 0 taken at h = 0): grad_val [rows][cols/tile][cap] (dtype)
 * receives lam rounded to the storage dtype in every used slot and +0 in the
 * padding; grad_dense [ovf_cap][cols] (dtype), when non-NULL, receives lam at
 * the active entries of the dense backup rows (r < min(n_ovf, ovf_cap)) and
 * +0 elsewhere.  With cnt, idx, ovf_rows and n_ovf of packed these buffers
 * form the gradient as a TwELL matrix.
 * Errors: INVALID_ARG, UNSUPPORTED (alignment), HIP.
 */
twell_status twell_l1_grad(const twell_matrix *packed, float lam, void *grad_val, void *grad_dense,
                           void *stream);

/*
 * twell_sparse_ffn_fused -- twell_sparse_ffn with the up and down projections
 * in ONE kernel: the single fused inference kernel of gist.science "Sparser,
 * Faster, Lighter Transformer Language Models", Resumen Técnico §2.B (up and
 * down from the TwELL gate activations in one flow, intermediates in
 * registers).  One wave per token computes v = h * (x_t . W_u^T[j]) for each
 * of its entries and adds v * W_d[j] to y_t in registers; overflow rows take
 * the dense fallback as in twell_sparse_ffn.  Same arguments, workspace
 * (twell_ffn_workspace_size) and results (within the same tolerance; the sum
 * order differs) as twell_sparse_ffn; d limited to 4096 (bf16) / 2048 (fp32).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
twell_status twell_sparse_ffn_fused(const twell_matrix *packed, const void *x, const void *w_gate, const void *w_up,
                                    const void *w_down, const float *gate_bias, void *y, int d, void *workspace,
                                    size_t ws_bytes, void *stream);

/*
 * twell_sparse_ffn_grouped -- the fused inference kernel in hidden-group-major
 * order (the same summary, §2.B), a measured prototype beside the two-kernel
 * route.  Hidden units are cut into groups of TwELL tiles whose w_up and
 * w_down rows together are about 4 MB (one XCD's L2; at most 16 groups), group
 * g placed on XCD g % 8.  The wave of (group, token) computes v = round(h * u)
 * for the token's entries in the group and adds v * W_d[j] into fp32
 * registers, then writes that partial output row; a second kernel adds the
 * groups' partial rows in group order (deterministic) and rounds y once.
 * Overflow rows take the dense fallback as in twell_sparse_ffn.  Same
 * arguments and results (within the same tolerance) as twell_sparse_ffn;
 * workspace: twell_sparse_ffn_grouped_workspace_size() bytes, which adds
 * n_groups * T * d fp32 partial rows (1 GiB at T = 8192, d = 2048, 16 groups)
 * to the forward's workspace; d limited to 4096 (bf16) / 2048 (fp32).
 * packed may be in either layout: with TWELL_LAYOUT_TILES (written so by
 * twell_gate_pack) a group's TwELL records are read tile by tile, each tile's
 * records of consecutive tokens contiguous.  The layout changes only where the
 * records are read from: y is bit for bit the same.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
size_t twell_sparse_ffn_grouped_workspace_size(int T, int d, int F, int tile, int cap, twell_dtype dtype);
twell_status twell_sparse_ffn_grouped(const twell_matrix *packed, const void *x, const void *w_gate,
                                      const void *w_up, const void *w_down, const float *gate_bias, void *y,
                                      int d, void *workspace, size_t ws_bytes, void *stream);

/*
 * twell_ffn_backward -- gradients of the ReLU-gated FFN layer from its
 * activations in the hybrid format (gist.science "Sparser, Faster, Lighter
 * Transformer Language Models", Resumen Técnico §2.A: the hybrid format keeps
 * the activations needed for back-propagation; §2.B: training kernels for
 * hybrid-times-dense and dense-times-hybrid products and the sparse
 * transpose).  With the forward y = (h * (x W_u^T)) W_d, h = ReLU(x W_g^T +
 * beta) as stored in `h`, the caller's upstream gradient dy and the L1 term
 * lam * ||h||_1, for every active entry (t, j) of h (u = x_t . W_u[j]):
 *     da = dy_t . W_d[j],   du = da * h,   dpre = da * u + lam
 *     dx_t    = sum_j du W_u[j] + dpre W_g[j]
 *     dW_u[j] = sum_t du x_t,  dW_g[j] = sum_t dpre x_t,  dW_d[j] = sum_t h u dy_t
 * The stored h is used as it is (the forward's rounding passed through as the
 * identity); ReLU's derivative is 1 on active entries and 0 elsewhere.  No
 * gradient is formed for the gate bias.
 *
 * h:      the activations (rows T, cols F, width, dtype); every dense row must
 *         be listed and stored: dense_cap >= *n_dense and dense non-NULL when
 *         dense_cap > 0 (a dense row that is not stored contributes nothing);
 *         dense 16-byte aligned when F is a multiple of 128.  h->u non-NULL:
 *         the ELL rows with a saved u take it from there instead of gathering
 *         W_u rows again (the others, and the dense rows, recompute it).
 * x, dy:  [T][d] dtype;  w_gate, w_up, w_down: [F][d] dtype (as the forward).
 * dx:     [T][d] dtype, overwritten (one rounding of fp32 sums).
 * dw_gate, dw_up, dw_down: [F][d] fp32, overwritten.
 * workspace: >= twell_ffn_backward_workspace_size(T, d, F, width, dense_cap,
 *         dtype) bytes, 256-byte aligned; about 28 bytes per entry slot.  With
 *         F a multiple of 128 the dense rows are computed with matrix-core
 *         matmuls (U = x W_u^T and DA = dy W_d^T over the listed rows, then
 *         dx and the weight gradients), there are T*width entry slots, and
 *         per dense row (2*s + 12)*F + 2*ns*s*d bytes of matmul operands
 *         (s = 2 and ns = 2 for bf16, s = 4 and ns = 1 for fp32) plus up to
 *         32 MB of split-K partial tiles; otherwise the
 *         dense rows' active entries are walked like the ELL rows', and there
 *         are T*width + dense_cap*F entry slots.
 * Sums run in a fixed order (deterministic); fp32 accumulation.  In the
 * dense rows' matmuls the dx product takes du and dpre rounded to the
 * storage dtype; the weight-gradient products take a, du and dpre as the sum
 * of two bf16 parts (high, and the rounded remainder) in bf16, as they are
 * in fp32.
 * Supported: bf16 d a multiple of 512 up to 4096, fp32 d a multiple of 256 up
 * to 2048; F <= 16384; T*d and F*d elements below 2 GiB of storage;
 * T*width + dense_cap*F < 2^31.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
size_t twell_ffn_backward_workspace_size(int T, int d, int F, int width, int dense_cap, twell_dtype dtype);
twell_status twell_ffn_backward(const twell_hybrid *h, const void *x, const void *w_gate, const void *w_up,
                                const void *w_down, const void *dy, float lam, int d, void *dx, float *dw_gate,
                                float *dw_up, float *dw_down, void *workspace, size_t ws_bytes, void *stream);

/*
 * twell_stream_probe -- streaming HBM probe (a measurement aid, not part of
 * the layer's computation; the pages define no such operation).
 *
 * mode 0: reads `bytes` from src, one 16-byte load per lane (a thread per
 *         chunk, grid-stride past 2^28 chunks); dst points at a 4-byte device sink that
 *         is written only if the XOR of everything read equals 0x9E3779B9.
 * mode 1: copies `bytes` from src to dst (the buffers must not overlap).
 * bytes / (time of the call) is the device's measured read (mode 0) or
 * copy (mode 1, count read + written bytes) bandwidth, the measured
 * denominator beside the 8 TB/s specification for HBM-bound kernels.
 * bytes == 0 launches nothing.
 * Errors: INVALID_ARG (NULL src/dst with bytes > 0, mode not 0 or 1),
 * UNSUPPORTED (bytes not a multiple of 16, src or dst not 16-byte aligned
 * (the sink: 4-byte aligned)), HIP.
 */
twell_status twell_stream_probe(const void *src, void *dst, size_t bytes, int mode, void *stream);

/*
 * twell_mfma_probe -- matrix-core issue-rate probe (a measurement aid, not
 * part of the layer's computation).
 *
 * Launches `blocks` workgroups of 512 threads (8 waves, two per SIMD); every
 * wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
 * register operands, with no memory traffic in the loop.  The call performs
 * 2*32*32*16 * 8 * iters * 8 * blocks flops; that ÷ the call's time is the
 * device's sustained bf16 matrix-core rate, the measured denominator beside
 * the 2.5 PFLOP/s specification for MFMA-bound kernels.  sink is a 4-byte
 * device buffer, written only if the accumulators sum to 1234567.
 * Errors: INVALID_ARG (NULL sink, iters < 1, blocks < 1), UNSUPPORTED (sink
 * not 4-byte aligned), HIP.
 */
twell_status twell_mfma_probe(float *sink, int iters, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
