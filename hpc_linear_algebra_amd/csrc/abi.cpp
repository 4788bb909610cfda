// extern "C" entry points declared in include/tlrgemm.h: argument checks,
// status codes and the thread-local error text around the planner/executor.
#include <exception>
#include <limits>
#include <new>
#include <string>

#include "tlr_plan.h"

struct tlr_plan {
  tlr::Plan p;
};

namespace tlr {

static thread_local std::string g_err;

void set_error(const std::string &msg) { g_err = msg; }

tlr_status fail(tlr_status s, const std::string &msg) {
  g_err = msg;
  return s;
}

}  // namespace tlr

#define TLR_GUARD(body)                                                      \
  try {                                                                      \
    body                                                                     \
  } catch (const std::bad_alloc &) {                                         \
    return tlr::fail(TLR_ERR_INVALID_ARG, "host allocation failed");         \
  } catch (const std::exception &e) {                                        \
    return tlr::fail(TLR_ERR_INVALID_ARG, std::string("exception: ") + e.what()); \
  } catch (...) {                                                            \
    return tlr::fail(TLR_ERR_INVALID_ARG, "unknown exception");              \
  }

extern "C" {

tlr_status tlr_gemm_analyze(tlr_dtype dt, tlr_op opA, const tlr_shape *A, tlr_op opB, const tlr_shape *B,
                            int64_t dense_rows, int64_t dense_cols, int64_t ldb, int64_t ldc,
                            size_t workspace_budget, int32_t n_streams, uint32_t flags, tlr_plan **plan_out) {
  TLR_GUARD({
    if (!plan_out) return tlr::fail(TLR_ERR_INVALID_ARG, "analyze: null plan_out");
    tlr_plan *h = new tlr_plan();
    tlr_status st = tlr::build_plan(dt, opA, A, opB, B, dense_rows, dense_cols, ldb, ldc, workspace_budget,
                                    n_streams, flags, true, &h->p);
    if (st != TLR_OK) {
      delete h;
      return st;
    }
    *plan_out = h;
    tlr::set_error("");
    return TLR_OK;
  })
}

tlr_status tlr_gemm_workspace_bytes(tlr_dtype dt, tlr_op opA, const tlr_shape *A, tlr_op opB, const tlr_shape *B,
                                    int64_t dense_rows, int64_t dense_cols, int32_t n_streams, uint32_t flags,
                                    int32_t runs, size_t *bytes_out) {
  TLR_GUARD({
    if (!bytes_out) return tlr::fail(TLR_ERR_INVALID_ARG, "workspace_bytes: null output");
    if (runs < 1) return tlr::fail(TLR_ERR_INVALID_ARG, "workspace_bytes: runs must be >= 1");
    const int64_t ld_b = std::max<int64_t>(1, dense_rows);
    int64_t mrows = 0;
    if (A) mrows = opA == TLR_OP_N ? A->rows : A->cols;
    else mrows = opA == TLR_OP_N ? dense_rows : dense_cols;   // dense A
    const int64_t ld_c = std::max<int64_t>(1, mrows);
    auto plan_at = [&](size_t budget, tlr::Plan &p) {
      return tlr::build_plan(dt, opA, A, opB, B, dense_rows, dense_cols, ld_b, ld_c, budget, n_streams, flags,
                             false, &p);
    };
    tlr::Plan full;
    tlr_status st = plan_at(0, full);
    if (st != TLR_OK) return st;
    size_t hi = full.ws_bytes;
    const int best_runs = (int)full.rects.size();
    const int target = std::max(runs, best_runs);
    // smallest budget whose schedule has at most `target` rectangles
    size_t lo = 0;  // infeasible or too many runs at lo (budget 0 would mean "unlimited")
    while (hi - lo > 1) {
      size_t mid = lo + (hi - lo) / 2;
      tlr::Plan p;
      tlr_status s2 = plan_at(mid, p);
      if (s2 == TLR_OK && (int)p.rects.size() <= target) hi = mid;
      else lo = mid;
    }
    *bytes_out = hi;
    tlr::set_error("");
    return TLR_OK;
  })
}

tlr_status tlr_plan_info(const tlr_plan *h, tlr_plan_summary *o) {
  if (!h || !o) return tlr::fail(TLR_ERR_INVALID_ARG, "plan_info: null argument");
  const tlr::Plan &p = h->p;
  o->m = p.m;
  o->n = p.n;
  o->k = p.k;
  o->useful_flops = p.useful_flops;
  o->executed_flops = p.executed_flops;
  o->flops_right = p.flops_right;
  o->flops_left = p.flops_left;
  o->final_flops_right = p.final_right;
  o->final_flops_left = p.final_left;
  o->algorithmic_bytes = p.alg_bytes;
  o->workspace_bytes = p.ws_bytes;
  o->descriptor_bytes = p.desc_bytes;
  o->runs = (int32_t)p.rects.size();
  o->groups = (int32_t)p.groups.size();
  o->launches = (int32_t)p.launches.size();
  o->dtype = (int32_t)p.dt;
  return TLR_OK;
}

tlr_status tlr_plan_rect(const tlr_plan *h, int32_t idx, int32_t *out, size_t *ws_bytes, double *flops) {
  if (!h || !out) return tlr::fail(TLR_ERR_INVALID_ARG, "plan_rect: null argument");
  const tlr::Plan &p = h->p;
  if (idx < 0 || idx >= (int32_t)p.rects.size()) return tlr::fail(TLR_ERR_INVALID_ARG, "plan_rect: index out of range");
  const tlr::Rect &r = p.rects[idx];
  out[0] = r.i0; out[1] = r.i1; out[2] = r.j0; out[3] = r.j1; out[4] = r.order; out[5] = r.group;
  if (ws_bytes) *ws_bytes = r.ws_bytes;
  if (flops) *flops = r.useful_flops;
  return TLR_OK;
}

tlr_status tlr_plan_stage_shapes(const tlr_plan *h, int32_t rect, int32_t stage, int64_t *mnk, int32_t cap,
                                 int32_t *count) {
  if (!h || !count || (cap > 0 && !mnk)) return tlr::fail(TLR_ERR_INVALID_ARG, "stage_shapes: null argument");
  const tlr::Plan &p = h->p;
  if (rect < 0 || rect >= (int32_t)p.rects.size()) return tlr::fail(TLR_ERR_INVALID_ARG, "stage_shapes: rect out of range");
  const tlr::Rect &r = p.rects[rect];
  const tlr::View &A = p.A;
  std::vector<int64_t> out;
  auto WJ = [&]() { int64_t w = 0; for (int j = r.j0; j < r.j1; ++j) w += p.ns[j]; return w; };
  auto WI = [&]() { int64_t w = 0; for (int i = r.i0; i < r.i1; ++i) w += A.rs[i]; return w; };
  if (stage == 1) {
    if (p.dense_b || p.dense_a) return tlr::fail(TLR_ERR_UNSUPPORTED, "stage_shapes: no coupling stage with a dense operand");
    for (int k = 0; k < A.qc; ++k) {
      int64_t M = 0, N = 0;
      for (int i = r.i0; i < r.i1; ++i) M += A.r(i, k);
      for (int j = r.j0; j < r.j1; ++j) N += p.B.r(k, j);
      out.insert(out.end(), {M, N, A.cs[k]});
    }
  } else if (stage == 3) {
    if (r.order == TLR_ORDER_RIGHT) {
      for (int i = r.i0; i < r.i1; ++i) {
        int64_t rho = 0;
        for (int k = 0; k < A.qc; ++k) rho += A.r(i, k);
        out.insert(out.end(), {A.rs[i], WJ(), rho});
      }
    } else {
      for (int j = r.j0; j < r.j1; ++j) {
        int64_t g = 0;
        for (int k = 0; k < A.qc; ++k) g += p.B.r(k, j);
        out.insert(out.end(), {WI(), p.ns[j], g});
      }
    }
  } else {
    return tlr::fail(TLR_ERR_INVALID_ARG, "stage_shapes: stage must be 1 or 3");
  }
  const int32_t n = (int32_t)(out.size() / 3);
  for (int32_t t = 0; t < std::min(n, cap); ++t)
    for (int c = 0; c < 3; ++c) mnk[3 * t + c] = out[3 * t + c];
  *count = n;
  return TLR_OK;
}

tlr_status tlr_plan_launch(const tlr_plan *h, int32_t idx, int32_t *oi, double *of) {
  if (!h || !oi || !of) return tlr::fail(TLR_ERR_INVALID_ARG, "plan_launch: null argument");
  const tlr::Plan &p = h->p;
  if (idx < 0 || idx >= (int32_t)p.launches.size()) return tlr::fail(TLR_ERR_INVALID_ARG, "plan_launch: index out of range");
  const tlr::Launch &L = p.launches[idx];
  oi[0] = L.stage;
  oi[1] = (int32_t)L.n_tasks;
  oi[2] = (int32_t)L.n_tiles;
  oi[3] = L.group;
  of[0] = L.useful_flops;
  of[1] = L.executed_flops;
  return TLR_OK;
}

tlr_status tlr_plan_destroy(tlr_plan *h) {
  TLR_GUARD({
    delete h;
    return TLR_OK;
  })
}

tlr_status tlr_plan_bind(tlr_plan *h, void *dev_desc, size_t bytes, void *stream) {
  if (!h) return tlr::fail(TLR_ERR_INVALID_ARG, "bind: null plan");
  TLR_GUARD({ return tlr::plan_bind(&h->p, dev_desc, bytes, stream); })
}

tlr_status tlr_gemm_execute(tlr_plan *h, double alpha, const tlr_buffers *A, const tlr_buffers *B,
                            const void *B_dense, int64_t ldb, double beta, void *C, int64_t ldc, void *workspace,
                            size_t workspace_bytes, void *const *streams, int32_t n_streams) {
  if (!h) return tlr::fail(TLR_ERR_INVALID_ARG, "execute: null plan");
  TLR_GUARD({
    return tlr::plan_execute(&h->p, alpha, A, B, B_dense, ldb, beta, C, ldc, workspace, workspace_bytes, streams,
                             n_streams);
  })
}

tlr_status tlr_gemm_execute_noalloc(tlr_plan *h, double alpha, const tlr_buffers *A, const tlr_buffers *B,
                                    const void *B_dense, int64_t ldb, double beta, void *C, int64_t ldc,
                                    void *const *streams, int32_t n_streams) {
  if (!h) return tlr::fail(TLR_ERR_INVALID_ARG, "execute_noalloc: null plan");
  TLR_GUARD({
    return tlr::plan_execute_noalloc(&h->p, alpha, A, B, B_dense, ldb, beta, C, ldc, streams, n_streams);
  })
}

tlr_status tlr_expand(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag, const int32_t *ranks_dev,
                      const tlr_buffers *X, double alpha, double beta, void *C, int64_t ldc, void *workspace,
                      size_t workspace_bytes, void *stream) {
  TLR_GUARD({
    return tlr::expand(dt, rows, cols, b, has_diag, ranks_dev, X, alpha, beta, C, ldc, workspace, workspace_bytes,
                       stream);
  })
}

tlr_status tlr_compress_workspace_bytes(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t max_rank,
                                        size_t *bytes_out) {
  TLR_GUARD({ return tlr::compress_workspace(dt, rows, cols, b, max_rank, bytes_out); })
}

tlr_status tlr_compress(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag, const void *X,
                        int64_t ldx, double tol, int32_t max_rank, const void *omega, int32_t *ranks_out, void *diag,
                        void *outer, void *inner, int64_t capacity, int32_t *info, void *workspace,
                        size_t workspace_bytes, void *stream) {
  TLR_GUARD({
    return tlr::compress(dt, rows, cols, b, has_diag, X, ldx, tol, max_rank, omega, ranks_out, diag, outer, inner,
                         capacity, info, workspace, workspace_bytes, stream);
  })
}

tlr_status tlr_compress_profile(int32_t max_calls) {
  TLR_GUARD({ return tlr::compress_profile(max_calls); })
}

tlr_status tlr_compress_profile_read(double *group_ms, int32_t *calls) {
  TLR_GUARD({ return tlr::compress_profile_read(group_ms, calls); })
}

tlr_status tlr_plan_profile(tlr_plan *h, int32_t max_executes) {
  if (!h) return tlr::fail(TLR_ERR_INVALID_ARG, "profile: null plan");
  TLR_GUARD({ return tlr::plan_profile(&h->p, max_executes); })
}

tlr_status tlr_plan_profile_read(tlr_plan *h, double *stage_ms, double *launch_ms, int32_t *executes) {
  if (!h || !stage_ms || !executes) return tlr::fail(TLR_ERR_INVALID_ARG, "profile_read: null argument");
  TLR_GUARD({ return tlr::plan_profile_read(&h->p, stage_ms, launch_ms, executes); })
}

tlr_status tlr_dense_gemm(tlr_dtype dt, tlr_op opA, tlr_op opB, int64_t m, int64_t n, int64_t k, double alpha,
                          const void *A, int64_t lda, const void *B, int64_t ldb, double beta, void *C, int64_t ldc,
                          void *stream) {
  TLR_GUARD({ return tlr::dense_gemm(dt, opA, opB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream); })
}

const char *tlr_status_string(tlr_status s) {
  switch (s) {
    case TLR_OK: return "TLR_OK";
    case TLR_ERR_INVALID_ARG: return "TLR_ERR_INVALID_ARG";
    case TLR_ERR_RANK: return "TLR_ERR_RANK";
    case TLR_ERR_WORKSPACE: return "TLR_ERR_WORKSPACE";
    case TLR_ERR_UNSUPPORTED: return "TLR_ERR_UNSUPPORTED";
    case TLR_ERR_HIP: return "TLR_ERR_HIP";
    case TLR_ERR_NOT_BOUND: return "TLR_ERR_NOT_BOUND";
  }
  return "TLR_ERR_UNKNOWN";
}

const char *tlr_last_error(void) { return tlr::g_err.c_str(); }

const char *tlr_version(void) { return "tlrgemm 0.1 (gfx950)"; }

}  // extern "C"
