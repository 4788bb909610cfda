/*
 * tlrgemm.h - Tile-Low-Rank GEMM with a dense output on AMD Instinct MI355X (gfx950).
 *
 *   C <- alpha * op(A) * op(B) + beta * C,   C dense, A TLR, B TLR or dense.
 *
 * The operation is the one stated in the introduction of "Tile-Low-Rank GEMM:
 * Designing Storage Around the Contraction" (dense C, one or both operands in
 * TLR format, op in {N, T}).  A TLR matrix is a regular grid of b x b tiles
 * (the last tile row / column is smaller when b does not divide the
 * dimension); diagonal tiles may be stored densely, every other tile (i,j) is
 * a factor pair U_ij V_ij^T of its own rank r_ij ("TLR Matrix
 * Multiplication", section "Introduction: TLR GEMM").
 *
 * Storage (section "Packing for the contraction" of the first page):
 *   outer  U: packed by tile row.  Column-major, leading dimension b.  Tile
 *             (i,j) occupies r_ij consecutive columns starting at column
 *             sum_{i'<i} rho_i' + sum_{j'<j} r_ij'      (rho_i = sum_j r_ij),
 *             of which its first s_i rows are used.
 *   inner  V: packed by tile column.  Column-major, leading dimension b.  Tile
 *             (i,j) occupies r_ij consecutive columns starting at column
 *             sum_{j'<j} kappa_j' + sum_{i'<i} r_i'j    (kappa_j = sum_i r_ij),
 *             of which its first s_j rows are used.
 *   diag   D: q slots of b*b elements; slot i holds tile (i,i) column-major
 *             with leading dimension b (top-left s_i x s_i used).  Only when
 *             the matrix is square and has_diag != 0; r_ii must then be 0.
 * Each tile takes exactly r_ij columns: no padding to a common rank.  Because
 * U is packed by tile row and V by tile column, a row panel of U and a column
 * panel of V are ordinary column-major matrices, which is what lets the
 * library fold tile indices into GEMM dimensions without copies.
 * op(X) = X^T is taken by swapping the roles of the two factor families and
 * the tile coordinates (section "Where fusion stops", Transposes); no data
 * moves.
 *
 * Dense matrices (C, a dense B) are column-major with a leading dimension.
 * All element types are float (TLR_F32), double (TLR_F64), IEEE half (TLR_F16)
 * or bfloat16 (TLR_BF16), the same for every buffer of one call.
 *
 * 16-bit types (the half-precision paths of the first page's evaluation, run
 * on the 16-bit matrix cores with float accumulation).  Every stored rank is
 * a multiple of 8: a tile of logical rank r is stored with its rank rounded up
 * to the next multiple of 8, the extra factor columns zero, which leaves the
 * product unchanged and keeps every factor column offset a multiple of 16
 * bytes (section "Packing for the contraction").  The tile size b, the
 * dimensions of A, B and C and the leading dimensions ldb and ldc are
 * multiples of 8 too, and every buffer is 16-byte aligned; analysis rejects
 * anything else with TLR_ERR_INVALID_ARG (TLR_ERR_RANK for a rank), execution
 * rejects a misaligned buffer.  The products are accumulated in float; each
 * workspace intermediate (the coupling blocks, the right or left products)
 * and C are rounded to the 16-bit type once, when written, and alpha and beta
 * are applied in float.  In half precision those intermediates must stay
 * within its range (|x| <= 65504; beyond it they become infinite); bfloat16
 * has float's range.
 *
 * Ownership: every device buffer (factors, diagonals, dense B, C, workspace,
 * descriptor buffer) belongs to the caller.  The library never allocates
 * device memory; the one piece it holds is the static workspace array of
 * tlr_gemm_execute_noalloc (TLR_STATIC_WORKSPACE_BYTES per GPU, part of the
 * loaded code object).  A plan owns host memory and the HIP events it
 * creates; the plan copies the rank tables at analysis time.
 *
 * Errors: every entry point returns a tlr_status and writes its outputs only
 * on TLR_OK.  tlr_last_error() returns a thread-local description of the most
 * recent failure.  Kernel faults are asynchronous and surface at the caller's
 * next synchronisation, as usual for HIP.
 *
 * Streams are passed as opaque pointers (hipStream_t values, e.g.
 * torch.cuda.Stream().cuda_stream under ROCm); NULL means the default stream.
 */
#ifndef TLRGEMM_H
#define TLRGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TLR_OK = 0,
  TLR_ERR_INVALID_ARG = -1,  /* null pointer, bad size, mismatched shapes or leading dims */
  TLR_ERR_RANK = -2,         /* r_ij < 0, r_ij > min(s_i, s_j), or r_ii != 0 with a dense diagonal */
  TLR_ERR_WORKSPACE = -3,    /* budget below what one output tile needs, or workspace too small */
  TLR_ERR_UNSUPPORTED = -4,  /* combination not provided (e.g. forcing the left order with a dense B) */
  TLR_ERR_HIP = -5,          /* a HIP runtime call failed */
  TLR_ERR_NOT_BOUND = -6     /* execute before tlr_plan_bind */
} tlr_status;

typedef enum { TLR_F32 = 0, TLR_F64 = 1, TLR_F16 = 2, TLR_BF16 = 3 } tlr_dtype;
typedef enum { TLR_OP_N = 0, TLR_OP_T = 1 } tlr_op;
typedef enum { TLR_ORDER_RIGHT = 0, TLR_ORDER_LEFT = 1 } tlr_order;

/* Flags of tlr_gemm_analyze / tlr_gemm_workspace_bytes. */
#define TLR_PLAN_FORCE_RIGHT 0x1u  /* every rectangle uses U (S Z^T) */
#define TLR_PLAN_FORCE_LEFT  0x2u  /* every rectangle uses (U S) Z^T (TLR x TLR only) */
#define TLR_PLAN_NO_REGIONS  0x4u  /* do not split boundary regions onto their own streams */
#define TLR_PLAN_VALIDATE    0x8u  /* also run the exhaustive descriptor self-check (slow; for tests) */
#define TLR_PLAN_PIPELINE    0x10u /* two arenas on two streams: stages 1-2 of one rectangle run beside
                                      stage 3 of the previous one (needs n_streams >= 2) */
#define TLR_PLAN_PER_K       0x20u /* the per-contraction-tile loop instead ("Many small GEMMs"): for
                                      each k, the coupling V_ik^T W_kj, the right product S Z_kj^T
                                      and the update C_ij += U_ik T of every output tile, one pass
                                      over C per k (TLR x TLR only; a comparator: with operands
                                      padded to one rank it is the batched-GEMM baseline the page
                                      compares against) */

/* Structure of one stored TLR operand (host data; no device pointers). */
typedef struct {
  int64_t rows, cols;      /* stored dimensions (before op) */
  int32_t b;               /* tile size, >= 1; q_r = ceil(rows/b), q_c = ceil(cols/b) */
  int32_t has_diag;        /* 1: diagonal tiles dense (rows == cols required) */
  const int32_t *ranks;    /* q_r*q_c ranks, column-major: rank of tile (i,j) at ranks[i + j*q_r] */
} tlr_shape;

/* Device buffers of one stored TLR operand, laid out as described above. */
typedef struct {
  const void *diag;        /* NULL iff has_diag == 0 */
  const void *outer;       /* U, packed by tile row;  may be NULL when every rank is 0 */
  const void *inner;       /* V, packed by tile column; may be NULL when every rank is 0 */
} tlr_buffers;

typedef struct tlr_plan tlr_plan;

/* Counts describing a plan (tlr_plan_info). */
typedef struct {
  int64_t m, n, k;             /* C is m x n; the contraction has k columns of op(A) */
  double useful_flops;         /* flops of the method for the chosen orders, from rank metadata */
  double executed_flops;       /* sum over kernel tasks of 2*M*N*K (>= useful when some ranks are 0) */
  double flops_right;          /* whole-C useful flops if every tile used the right order */
  double flops_left;           /* ... the left order (-1 for a dense B) */
  double final_flops_right;    /* 2 sum_i m_i rho_i sum_j n_j */
  double final_flops_left;     /* 2 sum_j n_j gamma_j sum_i m_i (-1 for a dense B) */
  double algorithmic_bytes;    /* compressed A + (compressed or dense) B + C written once (add m*n elements
                                  for the read of C when beta != 0) */
  size_t workspace_bytes;      /* device workspace execute needs (<= the analysis budget) */
  size_t descriptor_bytes;     /* device buffer size tlr_plan_bind needs */
  int32_t runs;                /* output rectangles */
  int32_t groups;              /* region groups (each on its own stream when streams allow) */
  int32_t launches;            /* kernel launches per execute */
  int32_t dtype;               /* tlr_dtype */
} tlr_plan_summary;

/* ---- host-only entry points (no HIP calls) --------------------------------- */

/*
 * tlr_gemm_analyze: build the plan of one product shape ("Association order and
 * workspace": rank prefixes, association order per rectangle, rectangles under
 * the workspace budget, grouped descriptors; reusable for every product with
 * the same rank structure).
 *   dt          element type of every buffer.
 *   opA, A      op and structure of A; A == NULL selects a dense A of
 *               dense_rows x dense_cols (stored, column-major, leading dim ldb):
 *               the dense x TLR product, evaluated in the left order with
 *               op(A) W in place of the coupling (at most one operand dense).
 *   opB, B      op and structure of B; B == NULL selects a dense B of
 *               dense_rows x dense_cols (stored, column-major, leading dim ldb).
 *   ldb         leading dimension of the dense operand (ignored when both are
 *               TLR; < 2^21).
 *   ldc         leading dimension of C (>= m).
 *   workspace_budget  bytes of device workspace execute may use; 0 means no limit.
 *   n_streams   streams execute will be given (>= 1); boundary regions of C
 *               (last tile row / column smaller than b) run concurrently when >= 2.
 *               With TLR_PLAN_PIPELINE the rectangles alternate between two
 *               workspace arenas and streams 0 and 1 ("Association order and
 *               workspace": rectangles write disjoint parts of C, so with two
 *               arenas and two streams the first stages of one rectangle can
 *               overlap the final GEMMs of the previous one, at twice the
 *               workspace); the budget then covers both arenas, and with no
 *               budget each arena is sized for a quarter of C.
 *   flags       TLR_PLAN_* bits.
 *   plan_out    receives a new plan (free with tlr_plan_destroy).
 * Every plan is checked before it is returned: each operand and output range a
 * kernel task can touch must lie inside the buffer sizes the layout above
 * implies (factor buffers b * sum(r_ij) elements, diagonal q*b*b, dense
 * operand ldb * cols, C ldc * n, workspace workspace_bytes); with TLR_PLAN_VALIDATE it
 * also checks that writes inside one launch never overlap, that every
 * workspace element a launch reads was written earlier for the same output
 * rectangle, and that each element of C is written exactly once.
 * Errors: TLR_ERR_INVALID_ARG (shapes, tile sizes or leading dims inconsistent),
 * TLR_ERR_RANK, TLR_ERR_WORKSPACE (budget below one output tile's needs),
 * TLR_ERR_UNSUPPORTED.
 */
tlr_status tlr_gemm_analyze(tlr_dtype dt, tlr_op opA, const tlr_shape *A,
                            tlr_op opB, const tlr_shape *B,
                            int64_t dense_rows, int64_t dense_cols, int64_t ldb,
                            int64_t ldc, size_t workspace_budget, int32_t n_streams,
                            uint32_t flags, tlr_plan **plan_out);

/*
 * tlr_gemm_workspace_bytes: the smallest budget whose schedule has at most
 * `runs` rectangles (runs >= 1; runs == 1 gives the budget of one rectangle
 * covering all of C), found by bisection over the scheduler
 * ("Association order and workspace": workspace bytes for a target number of
 * runs).  Arguments as for tlr_gemm_analyze.  Errors as for analyze.
 */
tlr_status tlr_gemm_workspace_bytes(tlr_dtype dt, tlr_op opA, const tlr_shape *A,
                                    tlr_op opB, const tlr_shape *B,
                                    int64_t dense_rows, int64_t dense_cols,
                                    int32_t n_streams, uint32_t flags, int32_t runs,
                                    size_t *bytes_out);

/* tlr_plan_info: fill *out.  Plumbing: the pages define no such call; the
 * counts are the rank arithmetic of "Association order and workspace" (useful
 * flops, final-stage costs F_R and F_L) and the sizes this library needs.
 * Errors: TLR_ERR_INVALID_ARG on NULL. */
tlr_status tlr_plan_info(const tlr_plan *p, tlr_plan_summary *out);

/*
 * tlr_plan_rect: rectangle `idx` (0 <= idx < runs) of the schedule
 * (introspection; the rectangles are those of "Association order and
 * workspace", the call itself is plumbing the pages do not define).
 *   out_i32[0..5] = first tile row, end tile row (exclusive), first tile
 *                   column, end tile column, order (tlr_order), group.
 *   ws_bytes      workspace the rectangle uses inside its group's arena.
 *   useful_flops  useful flops of the rectangle.
 */
tlr_status tlr_plan_rect(const tlr_plan *p, int32_t idx, int32_t *out_i32,
                         size_t *ws_bytes, double *useful_flops);

/*
 * tlr_plan_stage_shapes: (M, N, K) triples of the logical GEMMs of one stage of
 * rectangle `rect` (introspection, for checking the plan against the shapes
 * the GEMM page prints; the call is plumbing the pages do not define), in order:
 *   stage 1  one coupling GEMM per contraction tile k ("One product, three
 *            stages", Stage 1): (sum_{i in I} r_ik, sum_{j in J} r_kj, s_k);
 *   stage 3  the final GEMMs: per tile row i (right order) (m_i, sum_J n_j, rho_i),
 *            per tile column j (left order) (sum_I m_i, n_j, gamma_j).
 * Writes min(count, cap) triples to mnk[3*t..3*t+2]; *count = number available.
 */
tlr_status tlr_plan_stage_shapes(const tlr_plan *p, int32_t rect, int32_t stage,
                                 int64_t *mnk, int32_t cap, int32_t *count);

/*
 * tlr_plan_launch: launch `idx` (0 <= idx < launches) of one execute
 * (introspection; plumbing the pages do not define).
 *   out_i32[0..3] = stage, tasks, workgroups, group.  Stages: 1 coupling,
 *   2 right/left product, 3 final update, 4 the diagonal-term products that
 *   read only the inputs (X = op(D_A) W or X' = V^T op(D_B), and the op(D_A) W
 *   or op(D_B)^T V blocks of the terminal matrices; the "easy terms" of "TLR
 *   Matrix Multiplication"), run on a side stream beside stages 1 and 2.
 *   out_f64[0..1] = useful flops, executed flops of the launch.
 */
tlr_status tlr_plan_launch(const tlr_plan *p, int32_t idx, int32_t *out_i32, double *out_f64);

/* tlr_plan_destroy: free the plan and its events (NULL is accepted).  Plumbing:
 * the pages define no such call. */
tlr_status tlr_plan_destroy(tlr_plan *p);

/* ---- device entry points ------------------------------------------------- */

/*
 * tlr_plan_bind: copy the plan's descriptor tables into `dev_desc`, a caller
 * device buffer of at least descriptor_bytes bytes (256-byte aligned), on
 * `stream`, and create the plan's fork/join events on the current device.
 * The buffer must stay alive and unmodified while the plan is executed.
 * Plumbing the pages do not define: the GEMM page only says that this setup
 * is done once per rank structure and skipped afterwards ("Association order
 * and workspace").
 * Errors: TLR_ERR_INVALID_ARG (NULL, too small, misaligned), TLR_ERR_HIP.
 */
tlr_status tlr_plan_bind(tlr_plan *p, void *dev_desc, size_t bytes, void *stream);

/*
 * tlr_gemm_execute: C <- alpha op(A) op(B) + beta C with the bound plan: the
 * BLAS-style operation of the GEMM page's introduction, with a dense C and one
 * or both operands in TLR format ("Tile-Low-Rank GEMM: Designing Storage
 * Around the Contraction", introduction), evaluated in the three stages of
 * "One product, three stages" (coupling, right or left product, one update of
 * C with the sum over k inside the GEMM) and with the diagonal terms of "TLR
 * Matrix Multiplication", "Regular TLR GEMM".
 *   A, B        device buffers of the analysed TLR operands (NULL for the
 *               dense one).
 *   B_dense     the dense operand (dense A or dense B as analysed), leading
 *               dim ldb; NULL when both operands are TLR.
 *   C           m x n column-major, leading dim ldc (both as analysed).
 *   workspace   device buffer of at least workspace_bytes (256-byte aligned).
 *   streams     n_streams >= 1 streams; streams[0] is the caller's: the call is
 *               ordered after earlier work on streams[0] and later work on
 *               streams[0] is ordered after it.  Other streams are forked from
 *               and joined back to streams[0] with events.
 * beta == 0 never reads C (NaN in C does not propagate); alpha == 0 only scales C.
 * Asynchronous: no host synchronisation.
 * 16-bit types: every buffer (factors, diagonals, dense operand, C, workspace)
 * must be 16-byte aligned.
 * Errors: TLR_ERR_NOT_BOUND, TLR_ERR_INVALID_ARG (NULL buffers, ld mismatch,
 * a 16-bit buffer off a 16-byte boundary; nothing is launched),
 * TLR_ERR_WORKSPACE (workspace too small), TLR_ERR_HIP (launch failure).
 */
tlr_status tlr_gemm_execute(tlr_plan *p, double alpha,
                            const tlr_buffers *A, const tlr_buffers *B,
                            const void *B_dense, int64_t ldb,
                            double beta, void *C, int64_t ldc,
                            void *workspace, size_t workspace_bytes,
                            void *const *streams, int32_t n_streams);

/* Bytes of the static device workspace of tlr_gemm_execute_noalloc (per GPU). */
#define TLR_STATIC_WORKSPACE_BYTES (256u * 1024u * 1024u)

/*
 * tlr_gemm_execute_noalloc: tlr_gemm_execute without a workspace argument,
 * for callers that cannot allocate device memory at the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * same plan runs the same launches; the workspace is the library's own static
 * device array of TLR_STATIC_WORKSPACE_BYTES, one per GPU, which every GPU the
 * library runs on holds until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the plan must already
 * be bound (tlr_plan_bind, whose descriptor buffer the caller allocates once).
 * Every call on one GPU shares that GPU's array and leaves its last contents
 * in it (no product reads workspace it has not written first, so nothing
 * needs clearing).  Calls on one GPU must be ordered (one stream, or events
 * between them): calls that overlap race on the shared array.
 *   Arguments as for tlr_gemm_execute.
 * Errors: as tlr_gemm_execute; TLR_ERR_WORKSPACE when the plan needs more than
 * TLR_STATIC_WORKSPACE_BYTES (analyse with a budget at most that size);
 * nothing is launched then.
 */
tlr_status tlr_gemm_execute_noalloc(tlr_plan *p, double alpha,
                                    const tlr_buffers *A, const tlr_buffers *B,
                                    const void *B_dense, int64_t ldb,
                                    double beta, void *C, int64_t ldc,
                                    void *const *streams, int32_t n_streams);

/*
 * Profiling (plumbing the pages do not define; it feeds the measurement).
 * tlr_plan_profile: record a HIP event pair around every launch of the next
 * `max_executes` executes (0 switches recording off).  Creates the events on
 * the current device.  Errors: TLR_ERR_HIP.
 * tlr_plan_profile_read: after the caller has synchronised, sum the recorded
 * kernel time per stage into stage_ms[5]: stage_ms[0..2] = stages 1..3,
 * stage_ms[3] = the whole execute (first launch start to last launch end on
 * streams[0]), stage_ms[4] = stage 4 (the side launches, which overlap stages
 * 1 and 2);
 * launch_ms (may be NULL) receives the per-launch sums, `launches` entries.
 * *executes = executes recorded.  Resets the record.
 */
tlr_status tlr_plan_profile(tlr_plan *p, int32_t max_executes);
tlr_status tlr_plan_profile_read(tlr_plan *p, double *stage_ms, double *launch_ms,
                                 int32_t *executes);

/*
 * tlr_dense_gemm: C <- alpha op(A) op(B) + beta C for dense column-major
 * matrices, on the same MFMA kernel (one K segment per output tile).  It is
 * the same-chip dense reference the TLR product is compared with ("Results":
 * dense-GEMM time scaled by the ratio of executed flops).
 *   op(A) is m x k, op(B) is k x n, C is m x n; lda/ldb/ldc >= rows of the
 *   stored matrices, lda and ldb < 2^21.  beta == 0 never reads C.  No workspace.
 *   TLR_F32 and TLR_F64 only.
 * Errors: TLR_ERR_INVALID_ARG, TLR_ERR_UNSUPPORTED (a 16-bit type), TLR_ERR_HIP.
 */
tlr_status tlr_dense_gemm(tlr_dtype dt, tlr_op opA, tlr_op opB, int64_t m, int64_t n,
                          int64_t k, double alpha, const void *A, int64_t lda,
                          const void *B, int64_t ldb, double beta, void *C, int64_t ldc,
                          void *stream);

/* ---- TLR output: expansion and compression --------------------------------
 *
 * "TLR Matrix Multiplication", "Introduction: TLR GEMM": each of A, B and C
 * may be stored densely or in TLR format, and the TLR-output cases extend
 * the dense-output product.  The pages give no algorithm or accuracy target
 * for them; this library reads them as: the exact result tile, then every
 * off-diagonal tile replaced by its truncated SVD of the smallest rank whose
 * discarded part meets a relative Frobenius tolerance tol,
 *     ||X_ij - U_ij V_ij^T||_F <= tol ||X_ij||_F,
 * diagonal tiles kept dense.  A product C <- alpha op(A) op(B) + beta C with
 * a TLR C is then: tlr_expand of C into a dense m x n scratch (alpha = 1,
 * beta = 0; skipped when beta == 0), tlr_gemm_execute into that scratch with
 * the caller's alpha and beta, and tlr_compress of the scratch into the new
 * C.  Only TLR_F32 and TLR_F64; everything runs on `stream` with no host
 * synchronisation, and the ranks of a compressed result stay on the device
 * until the caller copies them.
 */

/*
 * tlr_expand: C <- alpha X + beta C, X the dense matrix of a stored TLR
 * operand (tile (i,j) = U_ij V_ij^T of rank r_ij, dense diagonal tiles when
 * has_diag), C dense rows x cols column-major with leading dim ldc >= rows.
 *   ranks_dev  DEVICE q_r x q_c int32 ranks, column-major (r_ii = 0 with a
 *              dense diagonal): the layout of X's packed factors (as for
 *              tlr_shape.ranks).
 *   X          device buffers of the operand.
 *   workspace  device, at least 16 * q_r * q_c bytes, 8-byte aligned (the
 *              factor offsets, computed on the device).
 * beta == 0 never reads C.  Errors: TLR_ERR_INVALID_ARG, TLR_ERR_WORKSPACE,
 * TLR_ERR_UNSUPPORTED (16-bit types), TLR_ERR_HIP.
 */
tlr_status tlr_expand(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag,
                      const int32_t *ranks_dev, const tlr_buffers *X, double alpha, double beta,
                      void *C, int64_t ldc, void *workspace, size_t workspace_bytes, void *stream);

/* tlr_compress_workspace_bytes: device workspace tlr_compress needs for a
 * rows x cols matrix, tile size b and ranks up to max_rank.  Host only.
 * Errors as for tlr_compress's argument checks. */
tlr_status tlr_compress_workspace_bytes(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b,
                                        int32_t max_rank, size_t *bytes_out);

/*
 * tlr_compress: the dense rows x cols matrix X (column-major, leading dim
 * ldx) as a TLR operand with tile size b: diagonal tiles dense (has_diag,
 * square X), every other tile (i,j) the truncated SVD of the smallest rank
 * r_ij <= max_rank with ||X_ij - U_ij V_ij^T||_F <= tol ||X_ij||_F.
 * Method: a range sketch X_ij Omega with s = max_rank + 8 samples, its QR,
 * the projection X_ij^T Q and its QR, and a one-sided Jacobi SVD of the
 * s x s core; the energy the sketch misses counts as discarded.  The rank is
 * decided on squared singular values, so tol must lie well above the square
 * root of the unit roundoff (fp64: tol >= 1e-7; fp32: tol >= 1e-3); for an
 * input of numerical rank above s - 8 the sketch may miss energy.
 *   omega      device b x s Gaussian sketch (column-major, leading dim b),
 *              drawn by the caller, s = max_rank + 8 (max_rank <= 56).
 *   ranks_out  device q_r x q_c int32, column-major: the new ranks (0 on a
 *              dense diagonal).
 *   diag       device q_r slots of b*b (when has_diag), as in the storage above.
 *   outer, inner  device factor buffers (leading dim b) of `capacity`
 *              columns each; tile (i,j) is written at the packed offsets of
 *              its new rank (U packed by tile row, V by tile column).  U has
 *              orthogonal columns of norms sigma_k, V orthonormal columns.
 *   info       device int32[6]: [0] columns used (sum of the new ranks),
 *              [1] tiles that did not meet tol within max_rank (their rank is
 *              max_rank), [2] 1 when [0] exceeds capacity (then no factor is
 *              written; ranks and diagonal are), [3] Jacobi pair visits
 *              (2 x 2 Gram blocks formed) and [4] Jacobi rotations summed over
 *              the tiles (the SVD's work, for measurement), [5] sketch basis
 *              columns kept, summed over the tiles (the range finder stops
 *              once the sketch shows the rest of a tile negligible; at most
 *              max_rank + 8 per tile); [0], [3], [4], [5] saturate at
 *              INT32_MAX.
 *   workspace  device, tlr_compress_workspace_bytes, 256-byte aligned.
 * Errors: TLR_ERR_INVALID_ARG, TLR_ERR_WORKSPACE, TLR_ERR_UNSUPPORTED (16-bit
 * types, max_rank > 56), TLR_ERR_HIP.
 */
tlr_status tlr_compress(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag,
                        const void *X, int64_t ldx, double tol, int32_t max_rank, const void *omega,
                        int32_t *ranks_out, void *diag, void *outer, void *inner, int64_t capacity,
                        int32_t *info, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Profiling of the compression (plumbing the pages do not define; it feeds the
 * measurement).  tlr_compress_profile: record a HIP event pair, on the call's
 * stream, around each kernel group of the next `max_calls` tlr_compress calls
 * of the process (0 switches recording off).  Errors: TLR_ERR_INVALID_ARG
 * (negative count).
 * tlr_compress_profile_read: after the caller has synchronised, sum the
 * recorded time per group into group_ms[9]: 0 tile norms, 1 sketch products
 * X_t Omega, 2 QR of the sketches, 3 projections X_t^T Q_t, 4 QR of the
 * projections, 5 Jacobi SVD and ranks, 6 factor products, 7 rank scan,
 * 8 packing; *calls = calls recorded.  Resets the record.  Errors:
 * TLR_ERR_HIP when an event has not completed.
 */
tlr_status tlr_compress_profile(int32_t max_calls);
tlr_status tlr_compress_profile_read(double *group_ms, int32_t *calls);

/* Static description of a status code (plumbing; the pages define no error
 * handling). */
const char *tlr_status_string(tlr_status s);
/* Thread-local detail of the last failure on this thread ("" if none; plumbing). */
const char *tlr_last_error(void);
/* Library version string (plumbing). */
const char *tlr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TLRGEMM_H */
