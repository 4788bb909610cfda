// Host-side plan of one TLR GEMM shape: operand views, schedule, descriptors.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "tlr_desc.h"
#include "tlrgemm.h"

namespace tlr {

constexpr int BM = 128;            // workgroup block rows of every grouped launch
constexpr int BN = 128;            // block columns: wide launches
constexpr int BN_NARROW = 64;      // block columns: narrow launches (see launch_bn)
constexpr int BW16 = 256;          // block rows and columns of the wide 16-bit launches (final update, large ones)
constexpr int STRIP_W = 512;        // block columns of a strip launch (right/left product, K <= 16)
constexpr int STRIP_K = 16;         // largest K of a strip task: one K stage of the kernel
constexpr int STRIP_K16 = 32;       // the same for 16-bit types: one k-step of their MFMA
constexpr size_t WS_ALIGN = 256;   // byte alignment of every workspace buffer
constexpr int NUM_XCD = 8;         // MI355X: workgroups go round-robin over 8 XCDs
constexpr int AUX_PER_GROUP = 3;   // auxiliary streams of a group: two for load modes, one side lane

// One operand after op: tile (i,j) of op(X) is Outer_ij Inner_ij^T, or the
// dense diagonal (transposed when op = T).
struct View {
  int qr = 0, qc = 0;
  int64_t b = 0;
  std::vector<int64_t> rs, cs, ro, co;   // tile sizes / start offsets of rows, cols
  std::vector<int32_t> R;                // ranks of op(X), R[i + j*qr]
  std::vector<int64_t> ocol, icol;       // first column of tile (i,j)'s outer / inner factor
  bool diag = false, diag_trans = false;
  uint8_t outer_base = 0, inner_base = 0, diag_base = 0;
  int32_t r(int i, int j) const { return R[(size_t)i + (size_t)j * qr]; }
  int64_t oc(int i, int j) const { return ocol[(size_t)i + (size_t)j * qr]; }
  int64_t ic(int i, int j) const { return icol[(size_t)i + (size_t)j * qr]; }
};

struct Rect {
  int i0, i1, j0, j1;
  int order;         // tlr_order
  int group;
  size_t ws_bytes;   // inside the group's arena
  double useful_flops;
};

// Stage 4 holds the products of the diagonal terms that read only the inputs
// (X = D W or X' = V^T D, and the D W / D^T V blocks of the terminal
// matrices).  It runs on the group's side stream, forked from the group's
// stream just before `fork_at` is enqueued, beside stages 1 and 2; the final
// update waits for it (or for the grouped stage-2 launch that follows it on
// the side stream, see Launch::on_side).
constexpr int STAGE_SIDE = 4;

struct Launch {
  int stage;         // 1, 2, 3, or STAGE_SIDE
  int group;
  int rect;
  int wait_launch;   // >= 0: this launch's stream first waits for that launch (another stream)
  int fork_at;       // side launch: the launch of the group's stream it forks before; else -1
  bool on_side;      // a stage-1-3 launch that runs on the group's side stream (after the side launch)
  int bm;            // block rows of the launch's workgroups (BM, or BW16 for a wide 16-bit launch)
  int bn;            // block columns (BN or BN_NARROW; BW16 with bm = BW16; STRIP_W for a strip launch)
  bool beta_one;     // a later pass of the per-k loop over C: its updates use beta = 1
  int64_t task_off;  // the launch's tasks are tasks[task_off, task_off + n_tasks)
  int64_t tile_off;  // first DevTile of the launch in the tile table
  int64_t n_tiles;   // workgroups launched (padded to a multiple of NUM_XCD)
  // the table is the concatenation of one sub-table per load mode (each a
  // multiple of NUM_XCD entries, possibly empty): mode m covers entries
  // [tile_off + mode_off[m], tile_off + mode_off[m] + mode_tiles[m])
  int64_t mode_off[NUM_LOAD_MODES];
  int64_t mode_tiles[NUM_LOAD_MODES];
  int64_t n_tasks;
  double useful_flops, executed_flops;
};

struct Group {
  int stream;        // index into the streams given to execute
  size_t arena_off;  // byte offset of the group's arena in the workspace
  size_t arena_bytes;
  std::vector<int> rects;
  std::vector<int> launches;
};

struct Plan {
  tlr_dtype dt = TLR_F64;
  int es = 8;
  bool dense_b = false;
  bool dense_a = false;        // dense A (and TLR B): the left order with no coupling stage
  int opA = 0;
  View A, B;                  // B unused (except sizes) for a dense B
  int opB = 0;
  int64_t m = 0, n = 0, k = 0;
  int64_t ldb = 0, ldc = 0;
  int64_t dense_rows = 0, dense_cols = 0;
  std::vector<int64_t> ns, no;    // C column tiles (B view columns, or b-wide for a dense B)
  size_t budget = 0;
  int n_streams = 1;
  uint32_t flags = 0;

  std::vector<Rect> rects;
  std::vector<Group> groups;
  std::vector<Launch> launches;
  std::vector<DevTask> tasks;
  std::vector<DevTile> tiles;
  std::vector<int64_t> coltab;

  size_t ws_bytes = 0;
  size_t task_bytes_off = 0, tile_bytes_off = 0, ctab_bytes_off = 0, desc_bytes = 0;
  double useful_flops = 0, executed_flops = 0;
  double flops_right = 0, flops_left = -1, final_right = 0, final_left = -1;
  double alg_bytes = 0;

  // device state (set by bind / profile)
  void *dev_desc = nullptr;
  int device = -1;
  std::vector<void *> join_events;   // hipEvent_t, one per group
  std::vector<void *> dep_events;    // hipEvent_t, one per launch (recorded only when awaited)
  void *fork_event = nullptr;
  // load-mode sub-launches of one launch run concurrently: two auxiliary
  // streams per group, and per launch with several non-empty sub-tables one
  // fork event and two join events (null otherwise); a third auxiliary stream
  // per group carries its side launches, forked by side_events[l] (null
  // unless l is a side launch) and joined at the group's end by side_join
  std::vector<void *> aux_streams;   // hipStream_t, AUX_PER_GROUP per group
  std::vector<void *> mode_events;   // hipEvent_t, 3 per launch
  std::vector<void *> side_events;   // hipEvent_t, 1 per launch
  std::vector<void *> side_join;     // hipEvent_t, 1 per group
  std::vector<std::vector<int>> forks_at;   // per launch: the side launches forked just before it
  int prof_max = 0, prof_count = 0;
  std::vector<void *> prof_events;   // 2 per launch per execute + 2 per execute (whole)
  ~Plan();
};

// One GEMM per tile of a regular tile grid, every tile of a launch the same
// kind (the per-tile products of dense-to-TLR compression).  Tile (i, j) has
// s_i = min(b, rows - i b) rows and s_j = min(b, cols - j b) columns; its
// index is t = i + j qr.  Each workgroup derives its tile's task from its own
// index, so no descriptor table is needed.  An operand's element offset is
//   off + (i b) f_ro + (j b) f_co + t f_t.
struct TileAddr {
  int64_t off, f_ro, f_co, f_t;
  int32_t ld;
  uint8_t base, trans;        // base id (tlr_desc.h); trans as in DevOperand
};
struct TileGemm {
  int32_t qr, qc;
  int64_t rows, cols, b;
  int32_t skip_diag;          // 1: tiles with i == j do nothing
  int32_t m_sel, k_sel;       // extent of M / K: 0 = s_i, 1 = s_j, 2 = n_fixed
  int32_t n;                  // N of every tile (<= 128)
  int32_t n_fixed;
  TileAddr a, bop, c;         // A (M x K), B (K x N), C (M x N, trans ignored)
};

// Planner (host only).
tlr_status build_plan(tlr_dtype dt, tlr_op opA, const tlr_shape *A, tlr_op opB,
                      const tlr_shape *B, int64_t dense_rows, int64_t dense_cols,
                      int64_t ldb, int64_t ldc, size_t budget, int n_streams,
                      uint32_t flags, bool build_descriptors, Plan *out);

// Executor (HIP runtime).
tlr_status plan_bind(Plan *p, void *dev_desc, size_t bytes, void *stream);
tlr_status plan_execute(Plan *p, double alpha, const tlr_buffers *A, const tlr_buffers *B,
                        const void *B_dense, int64_t ldb, double beta, void *C, int64_t ldc,
                        void *ws, size_t ws_bytes, void *const *streams, int n_streams);
tlr_status plan_execute_noalloc(Plan *p, double alpha, const tlr_buffers *A, const tlr_buffers *B,
                                const void *B_dense, int64_t ldb, double beta, void *C, int64_t ldc,
                                void *const *streams, int n_streams);
tlr_status expand(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag, const int32_t *ranks,
                  const tlr_buffers *X, double alpha, double beta, void *C, int64_t ldc, void *ws, size_t ws_bytes,
                  void *stream);
tlr_status compress_workspace(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t max_rank, size_t *bytes);
constexpr int COMPRESS_PROFILE_GROUPS = 9;
tlr_status compress_profile(int32_t max_calls);
tlr_status compress_profile_read(double *group_ms, int32_t *calls);
tlr_status compress(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag, const void *X, int64_t ldx,
                    double tol, int32_t max_rank, const void *omega, int32_t *ranks_out, void *diag, void *outer,
                    void *inner, int64_t capacity, int32_t *info, void *ws, size_t ws_bytes, void *stream);
tlr_status plan_profile(Plan *p, int max_exec);
tlr_status plan_profile_read(Plan *p, double *stage_ms, double *launch_ms, int32_t *execs);
void plan_release_device(Plan *p);
tlr_status dense_gemm(tlr_dtype dt, tlr_op opA, tlr_op opB, int64_t m, int64_t n, int64_t k,
                      double alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                      double beta, void *C, int64_t ldc, void *stream);

// Kernel launchers (gemm.hip).
int launch_grouped(tlr_dtype dt, int stage, int mode, int bn, const DevTask *tasks, const DevTile *tiles,
                   int64_t n_tiles, const int64_t *coltab, const Bases &bases, double alpha, double beta,
                   void *stream);
int launch_single(tlr_dtype dt, int mode, const DevTask &task, const Bases &bases, double alpha,
                  double beta, void *stream);
int launch_scale(tlr_dtype dt, void *C, int64_t m, int64_t n, int64_t ldc, double beta,
                 void *stream);
int launch_tile_gemm(tlr_dtype dt, int mode, const TileGemm &g, const Bases &bases, void *stream);
// 16-bit types (gemm16.hip); launch_grouped and launch_scale forward to these.
int launch_grouped16(tlr_dtype dt, int stage, int bn, const DevTask *tasks, const DevTile *tiles,
                     int64_t n_tiles, const int64_t *coltab, const Bases &bases, double alpha, double beta,
                     void *stream);
int launch_scale16(tlr_dtype dt, void *C, int64_t m, int64_t n, int64_t ldc, double beta, void *stream);

// Error reporting.
void set_error(const std::string &msg);
tlr_status fail(tlr_status s, const std::string &msg);

}  // namespace tlr
