// Host planner of the TLR GEMM: operand views, association order, rectangles
// under a workspace budget, and the descriptor tables of every launch.
//
// The method follows "Tile-Low-Rank GEMM: Designing Storage Around the
// Contraction" (sections "One product, three stages", "Where fusion stops",
// "Association order and workspace") with the dense-diagonal and boundary
// handling of "TLR Matrix Multiplication" ("Regular TLR GEMM", boundary
// decomposition, "Output traversal and workspace budget").  No HIP calls here.
//
// Per output rectangle (I, J) the right order U (S Z^T) runs
//   launch 1: S_k = V_{I,k}^T W_{k,J} for every contraction tile k (coupling,
//             one GEMM per k with i fused into M and j into N), and the
//             diagonal-term products X_i = D_A,ii W_{i,J};
//   launch 2: for every (k, j): the right product S_ikj Z_kj^T for all i in I at
//             once (or V_ij^T D_B,jj when k = j is a dense diagonal tile),
//             written through an indirect column map straight into row block k
//             of every terminal matrix T_i (stored transposed, W_J x rho_i);
//   launch 3: for every output tile (i, j): C_ij = alpha (U_i T_i[:, j] + X_ij Z_ij^T
//             or D_A,ii D_B,ii) + beta C_ij, so the whole sum over k is the GEMM
//             reduction and C is read and written once.
// The left order (U S) Z^T mirrors it with terminal matrices Y_j (W_I x gamma_j)
// and the diagonal-term products X'_j = V_{I,j}^T D_B,jj.
#include <algorithm>
#include <cstring>
#include <limits>
#include <numeric>

#include "tlr_plan.h"

namespace tlr {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
static int64_t even_up(int64_t x) { return x + (x & 1); }

static void split_dim(int64_t n, int64_t b, std::vector<int64_t> &s, std::vector<int64_t> &o) {
  s.clear();
  o.clear();
  if (n <= 0) return;
  int64_t q = ceil_div(n, b);
  for (int64_t t = 0; t < q; ++t) {
    o.push_back(t * b);
    s.push_back(std::min<int64_t>(b, n - t * b));
  }
}

// Validate a stored operand and build the view of op(X).  Factor offsets follow
// the packing rules: outer by tile row, inner by tile column, r_ij columns each.
static tlr_status make_view(const tlr_shape *X, int op, uint8_t outer_id, uint8_t inner_id,
                            uint8_t diag_id, const char *name, View *v) {
  if (!X) return fail(TLR_ERR_INVALID_ARG, std::string(name) + ": null shape");
  if (X->rows < 0 || X->cols < 0 || X->b < 1)
    return fail(TLR_ERR_INVALID_ARG, std::string(name) + ": bad rows/cols/b");
  if (X->has_diag && X->rows != X->cols)
    return fail(TLR_ERR_INVALID_ARG, std::string(name) + ": a dense diagonal needs a square matrix");
  if ((int64_t)X->b > (int64_t)std::numeric_limits<int32_t>::max() / 2)
    return fail(TLR_ERR_INVALID_ARG, std::string(name) + ": tile size too large");
  std::vector<int64_t> srs, sro, scs, sco;
  split_dim(X->rows, X->b, srs, sro);
  split_dim(X->cols, X->b, scs, sco);
  const int qr = (int)srs.size(), qc = (int)scs.size();
  if ((int64_t)qr * qc > 0 && !X->ranks) return fail(TLR_ERR_INVALID_ARG, std::string(name) + ": null ranks");
  std::vector<int32_t> R((size_t)qr * qc);
  for (int j = 0; j < qc; ++j)
    for (int i = 0; i < qr; ++i) {
      int32_t r = X->ranks[(size_t)i + (size_t)j * qr];
      if (r < 0 || r > std::min(srs[i], scs[j]))
        return fail(TLR_ERR_RANK, std::string(name) + ": rank out of range at tile (" +
                                      std::to_string(i) + "," + std::to_string(j) + ")");
      if (X->has_diag && i == j && r != 0)
        return fail(TLR_ERR_RANK, std::string(name) + ": diagonal tile rank must be 0 with a dense diagonal");
      R[(size_t)i + (size_t)j * qr] = r;
    }
  // stored offsets
  std::vector<int64_t> so((size_t)qr * qc), si((size_t)qr * qc);
  int64_t acc = 0;
  for (int i = 0; i < qr; ++i)
    for (int j = 0; j < qc; ++j) {
      so[(size_t)i + (size_t)j * qr] = acc;
      acc += R[(size_t)i + (size_t)j * qr];
    }
  acc = 0;
  for (int j = 0; j < qc; ++j)
    for (int i = 0; i < qr; ++i) {
      si[(size_t)i + (size_t)j * qr] = acc;
      acc += R[(size_t)i + (size_t)j * qr];
    }
  v->b = X->b;
  v->diag = X->has_diag != 0;
  v->diag_base = diag_id;
  if (op == TLR_OP_N) {
    v->qr = qr; v->qc = qc;
    v->rs = srs; v->ro = sro; v->cs = scs; v->co = sco;
    v->R = R; v->ocol = so; v->icol = si;
    v->outer_base = outer_id; v->inner_base = inner_id;
    v->diag_trans = false;
  } else {
    // tile (i,j) of X^T is V_ji U_ji^T: the inner family becomes the outer one
    v->qr = qc; v->qc = qr;
    v->rs = scs; v->ro = sco; v->cs = srs; v->co = sro;
    v->R.assign((size_t)qc * qr, 0);
    v->ocol.assign((size_t)qc * qr, 0);
    v->icol.assign((size_t)qc * qr, 0);
    for (int i = 0; i < qc; ++i)
      for (int j = 0; j < qr; ++j) {
        size_t d = (size_t)i + (size_t)j * qc, s = (size_t)j + (size_t)i * qr;
        v->R[d] = R[s];
        v->ocol[d] = si[s];
        v->icol[d] = so[s];
      }
    v->outer_base = inner_id; v->inner_base = outer_id;
    v->diag_trans = true;
  }
  return TLR_OK;
}

// ---------------------------------------------------------------------------
// Rank prefix sums used by the accounting.
struct Sums {
  int qm = 0, qk = 0, qn = 0;
  std::vector<int64_t> cumA;   // cumA[k*(qm+1) + i] = sum_{i'<i} RA(i',k)
  std::vector<int64_t> cumB;   // cumB[k*(qn+1) + j] = sum_{j'<j} RB(k,j')
  std::vector<int64_t> rho, gam;
  int64_t kap(int k, int i0, int i1) const { return cumA[(size_t)k * (qm + 1) + i1] - cumA[(size_t)k * (qm + 1) + i0]; }
  int64_t bet(int k, int j0, int j1) const { return cumB[(size_t)k * (qn + 1) + j1] - cumB[(size_t)k * (qn + 1) + j0]; }
};

static void build_sums(const Plan &p, Sums &s) {
  s.qm = p.A.qr;
  s.qk = p.A.qc;
  s.qn = (int)p.ns.size();
  s.cumA.assign((size_t)s.qk * (s.qm + 1), 0);
  for (int k = 0; k < s.qk; ++k)
    for (int i = 0; i < s.qm; ++i)
      s.cumA[(size_t)k * (s.qm + 1) + i + 1] = s.cumA[(size_t)k * (s.qm + 1) + i] + p.A.r(i, k);
  s.rho.assign(s.qm, 0);
  for (int i = 0; i < s.qm; ++i)
    for (int k = 0; k < s.qk; ++k) s.rho[i] += p.A.r(i, k);
  if (!p.dense_b) {
    s.cumB.assign((size_t)s.qk * (s.qn + 1), 0);
    for (int k = 0; k < s.qk; ++k)
      for (int j = 0; j < s.qn; ++j)
        s.cumB[(size_t)k * (s.qn + 1) + j + 1] = s.cumB[(size_t)k * (s.qn + 1) + j] + p.B.r(k, j);
    s.gam.assign(s.qn, 0);
    for (int j = 0; j < s.qn; ++j)
      for (int k = 0; k < s.qk; ++k) s.gam[j] += p.B.r(k, j);
  }
}

static int64_t width(const Plan &p, int j0, int j1) {
  return j1 > j0 ? p.no[j1 - 1] + p.ns[j1 - 1] - p.no[j0] : 0;
}
static int64_t height(const Plan &p, int i0, int i1) {
  return i1 > i0 ? p.A.ro[i1 - 1] + p.A.rs[i1 - 1] - p.A.ro[i0] : 0;
}

// Exact workspace bytes of one rectangle in one order (every buffer 256-B aligned).
// Coupling block S_k (kappa x beta) in the workspace: column-major S for the
// right order, S^T for the left, each with its leading dimension rounded up to
// even, so that the right or left product reads it with pair loads.
static int64_t s_ld(int64_t kappa, int64_t beta, int order) {
  return even_up(order == TLR_ORDER_RIGHT ? kappa : beta);
}
static int64_t s_elems(int64_t kappa, int64_t beta, int order) {
  return s_ld(kappa, beta, order) * (order == TLR_ORDER_RIGHT ? beta : kappa);
}

static size_t rect_ws(const Plan &p, const Sums &s, int i0, int i1, int j0, int j1, int order) {
  const size_t es = p.es;
  size_t tot = 0;
  const int64_t WJ = width(p, j0, j1), WI = height(p, i0, i1);
  if (p.dense_b) {
    for (int i = i0; i < i1; ++i)
      if (s.rho[i] > 0) tot += align_up((size_t)WJ * s.rho[i] * es, WS_ALIGN);
    return tot;
  }
  if (p.dense_a) {   // Y_j only
    for (int j = j0; j < j1; ++j)
      if (s.gam[j] > 0) tot += align_up((size_t)WI * s.gam[j] * es, WS_ALIGN);
    return tot;
  }
  for (int k = 0; k < s.qk; ++k) {
    int64_t M = s.kap(k, i0, i1), N = s.bet(k, j0, j1);
    if (M > 0 && N > 0) tot += align_up((size_t)s_elems(M, N, order) * es, WS_ALIGN);
  }
  if (order == TLR_ORDER_RIGHT) {
    for (int i = i0; i < i1; ++i) {
      if (s.rho[i] > 0) tot += align_up((size_t)WJ * s.rho[i] * es, WS_ALIGN);
      if (p.A.diag) {
        int64_t bi = s.bet(i, j0, j1);
        if (bi > 0) tot += align_up((size_t)p.A.rs[i] * bi * es, WS_ALIGN);
      }
    }
  } else {
    for (int j = j0; j < j1; ++j) {
      if (s.gam[j] > 0) tot += align_up((size_t)WI * s.gam[j] * es, WS_ALIGN);
      if (p.B.diag) {
        int64_t kj = s.kap(j, i0, i1);
        if (kj > 0) tot += align_up((size_t)kj * p.ns[j] * es, WS_ALIGN);
      }
    }
  }
  return tot;
}

// Useful flops of one rectangle in one order (terms with a zero rank count 0).
static double rect_useful(const Plan &p, const Sums &s, int i0, int i1, int j0, int j1, int order) {
  const View &A = p.A;
  double F = 0;
  const double WJ = (double)width(p, j0, j1);
  if (p.dense_b) {
    for (int k = 0; k < s.qk; ++k) F += 2.0 * WJ * A.cs[k] * s.kap(k, i0, i1);
    for (int i = i0; i < i1; ++i) {
      F += 2.0 * A.rs[i] * WJ * s.rho[i];
      if (A.diag) F += 2.0 * A.rs[i] * (double)A.rs[i] * WJ;
    }
    return F;
  }
  const View &B = p.B;
  if (p.dense_a) {
    // Y_j = op(A)[I, k-block] W_kj for every k; then Y_j Z_j^T, and op(A)[I, j-block] op(D_B,jj)
    const double WI = (double)height(p, i0, i1);
    for (int k = 0; k < s.qk; ++k) F += 2.0 * WI * A.cs[k] * s.bet(k, j0, j1);
    for (int j = j0; j < j1; ++j) {
      F += 2.0 * WI * (double)p.ns[j] * s.gam[j];
      if (B.diag) F += 2.0 * WI * (double)p.ns[j] * p.ns[j];
    }
    return F;
  }
  for (int k = 0; k < s.qk; ++k) F += 2.0 * s.kap(k, i0, i1) * s.bet(k, j0, j1) * A.cs[k];
  if (order == TLR_ORDER_RIGHT) {
    if (A.diag)
      for (int i = i0; i < i1; ++i) F += 2.0 * A.rs[i] * (double)A.rs[i] * s.bet(i, j0, j1);
    for (int k = 0; k < s.qk; ++k)
      for (int j = j0; j < j1; ++j) {
        if (B.diag && k == j) F += 2.0 * p.ns[j] * (double)p.ns[j] * s.kap(j, i0, i1);
        else F += 2.0 * p.ns[j] * (double)s.kap(k, i0, i1) * B.r(k, j);
      }
    for (int i = i0; i < i1; ++i)
      for (int j = j0; j < j1; ++j) {
        int64_t kk = 0;
        for (int k = 0; k < s.qk; ++k)
          if (B.r(k, j) > 0 || (B.diag && k == j)) kk += A.r(i, k);
        F += 2.0 * A.rs[i] * (double)p.ns[j] * kk;
        if (A.diag) {
          if (B.diag && i == j) F += 2.0 * A.rs[i] * (double)A.rs[i] * A.rs[i];
          else F += 2.0 * A.rs[i] * (double)p.ns[j] * B.r(i, j);
        }
      }
  } else {
    if (B.diag)
      for (int j = j0; j < j1; ++j) F += 2.0 * s.kap(j, i0, i1) * (double)p.ns[j] * p.ns[j];
    for (int i = i0; i < i1; ++i)
      for (int k = 0; k < s.qk; ++k) {
        if (A.diag && k == i) F += 2.0 * A.rs[i] * (double)A.rs[i] * s.bet(i, j0, j1);
        else F += 2.0 * A.rs[i] * (double)s.bet(k, j0, j1) * A.r(i, k);
      }
    for (int i = i0; i < i1; ++i)
      for (int j = j0; j < j1; ++j) {
        int64_t kk = 0;
        for (int k = 0; k < s.qk; ++k)
          if (A.r(i, k) > 0 || (A.diag && k == i)) kk += B.r(k, j);
        F += 2.0 * A.rs[i] * (double)p.ns[j] * kk;
        if (B.diag) {
          if (A.diag && i == j) F += 2.0 * A.rs[i] * (double)A.rs[i] * A.rs[i];
          else F += 2.0 * A.rs[i] * (double)p.ns[j] * A.r(i, j);
        }
      }
  }
  return F;
}

static bool order_allowed(const Plan &p, int order) {
  if (p.dense_b) return order == TLR_ORDER_RIGHT;
  if (p.dense_a) return order == TLR_ORDER_LEFT;
  if (p.flags & TLR_PLAN_FORCE_RIGHT) return order == TLR_ORDER_RIGHT;
  if (p.flags & TLR_PLAN_FORCE_LEFT) return order == TLR_ORDER_LEFT;
  return true;
}

static size_t min_ws(const Plan &p, const Sums &s, int i0, int i1, int j0, int j1) {
  size_t best = std::numeric_limits<size_t>::max();
  for (int o = 0; o < 2; ++o)
    if (order_allowed(p, o)) best = std::min(best, rect_ws(p, s, i0, i1, j0, j1, o));
  return best;
}

struct Region { int i0, i1, j0, j1; };

// Widest feasible block of tile columns, then the longest runs of tile rows
// that fit, then the cheaper feasible order of each rectangle.
static tlr_status schedule_region(const Plan &p, const Sums &s, const Region &g, size_t budget,
                                  int group, std::vector<Rect> &out) {
  auto fits = [&](int i0, int i1, int j0, int j1) { return min_ws(p, s, i0, i1, j0, j1) <= budget; };
  int jc = g.j0;
  while (jc < g.j1) {
    auto J_ok = [&](int je) {
      for (int i = g.i0; i < g.i1; ++i)
        if (!fits(i, i + 1, jc, je)) return false;
      return true;
    };
    if (!J_ok(jc + 1))
      return fail(TLR_ERR_WORKSPACE, "workspace budget " + std::to_string(budget) +
                                         " B is below what one output tile needs");
    int je = jc + 1;
    while (je < g.j1 && J_ok(je + 1)) ++je;
    int ic = g.i0;
    while (ic < g.i1) {
      int ie = ic + 1;
      while (ie < g.i1 && fits(ic, ie + 1, jc, je)) ++ie;
      Rect r{ic, ie, jc, je, -1, group, 0, 0};
      double bestF = 0;
      for (int o = 0; o < 2; ++o) {
        if (!order_allowed(p, o)) continue;
        size_t w = rect_ws(p, s, ic, ie, jc, je, o);
        if (w > budget) continue;
        double F = rect_useful(p, s, ic, ie, jc, je, o);
        if (r.order < 0 || F < bestF) { r.order = o; bestF = F; r.ws_bytes = w; }
      }
      r.useful_flops = bestF;
      out.push_back(r);
      ic = ie;
    }
    jc = je;
  }
  return TLR_OK;
}

// Split C into disjoint regions (interior, boundary column, boundary row,
// corner) when the last tile row / column is a remainder, so they can run on
// separate streams ("TLR Matrix Multiplication", four output regions).
static std::vector<Region> make_regions(const Plan &p, bool split) {
  const int qm = p.A.qr, qn = (int)p.ns.size();
  std::vector<Region> regs;
  if (qm == 0 || qn == 0) return regs;
  const bool rrem = split && qm > 1 && p.A.rs.back() < p.A.b;
  const bool crem = split && qn > 1 && p.ns.back() < p.A.b;
  const int mi = rrem ? qm - 1 : qm, mj = crem ? qn - 1 : qn;
  regs.push_back({0, mi, 0, mj});
  if (crem) regs.push_back({0, mi, mj, qn});
  if (rrem) regs.push_back({mi, qm, 0, mj});
  if (rrem && crem) regs.push_back({mi, qm, mj, qn});
  return regs;
}

// Rectangle pipelining: the schedule of one arena's budget, rectangles dealt
// alternately to two groups (streams 0 and 1) with an arena each.
static tlr_status schedule_pipelined(Plan &p, const Sums &s) {
  const Region whole{0, p.A.qr, 0, (int)p.ns.size()};
  size_t per_arena;
  if (p.budget) {
    per_arena = p.budget / 2 / WS_ALIGN * WS_ALIGN;
  } else {
    // no limit: the smallest arena for which C splits into at most 4 rectangles
    std::vector<Rect> rr;
    size_t hi = min_ws(p, s, whole.i0, whole.i1, whole.j0, whole.j1), lo = 0;
    while (hi - lo > WS_ALIGN) {
      size_t mid = lo + (hi - lo) / 2;
      rr.clear();
      if (schedule_region(p, s, whole, mid, 0, rr) == TLR_OK && rr.size() <= 4) hi = mid;
      else lo = mid;
    }
    per_arena = hi;
  }
  std::vector<Rect> rr;
  tlr_status st = schedule_region(p, s, whole, per_arena, 0, rr);
  if (st != TLR_OK) return st;
  p.rects = rr;
  for (int g = 0; g < 2; ++g) {
    Group G;
    G.stream = g;
    size_t mx = 0;
    for (size_t r = g; r < p.rects.size(); r += 2) {
      p.rects[r].group = g;
      G.rects.push_back((int)r);
      mx = std::max(mx, p.rects[r].ws_bytes);
    }
    G.arena_bytes = align_up(mx, WS_ALIGN);
    G.arena_off = g == 0 ? 0 : p.groups[0].arena_bytes;
    if (!G.rects.empty()) p.groups.push_back(G);
  }
  p.ws_bytes = 0;
  for (auto &G : p.groups) p.ws_bytes += G.arena_bytes;
  set_error("");
  return TLR_OK;
}

static tlr_status schedule(Plan &p, const Sums &s) {
  const size_t budget = p.budget ? p.budget : std::numeric_limits<size_t>::max();
  p.rects.clear();
  p.groups.clear();
  if (p.flags & TLR_PLAN_PIPELINE) {
    if (p.A.qr == 0 || p.ns.empty()) return TLR_OK;
    return schedule_pipelined(p, s);
  }
  const bool concurrent = p.n_streams >= 2 && !(p.flags & TLR_PLAN_NO_REGIONS);
  std::vector<Region> regs = make_regions(p, concurrent);
  if (regs.empty()) return TLR_OK;
  if (regs.size() > 1) {
    // boundary regions get what one run each needs, capped at a quarter of the budget
    std::vector<size_t> need(regs.size(), 0);
    size_t bsum = 0;
    for (size_t g = 1; g < regs.size(); ++g) {
      need[g] = align_up(min_ws(p, s, regs[g].i0, regs[g].i1, regs[g].j0, regs[g].j1), WS_ALIGN);
      bsum += need[g];
    }
    bool ok = true;
    std::vector<size_t> share(regs.size(), 0);
    if (budget == std::numeric_limits<size_t>::max()) {
      for (size_t g = 1; g < regs.size(); ++g) share[g] = need[g];
      share[0] = budget;
    } else {
      size_t cap = budget / 4;
      size_t used = 0;
      for (size_t g = 1; g < regs.size(); ++g) {
        share[g] = bsum <= cap ? need[g]
                               : (size_t)((double)cap * (double)need[g] / (double)bsum) / WS_ALIGN * WS_ALIGN;
        used += share[g];
      }
      share[0] = budget > used ? budget - used : 0;
    }
    std::vector<Rect> rects;
    for (size_t g = 0; g < regs.size() && ok; ++g) {
      std::vector<Rect> rr;
      tlr_status st = schedule_region(p, s, regs[g], share[g], (int)g, rr);
      if (st != TLR_OK) { ok = false; break; }
      rects.insert(rects.end(), rr.begin(), rr.end());
    }
    if (ok) {
      p.rects = rects;
      size_t off = 0;
      for (size_t g = 0; g < regs.size(); ++g) {
        Group G;
        G.stream = (int)(g % (size_t)p.n_streams);
        G.arena_off = off;
        size_t mx = 0;
        for (size_t r = 0; r < p.rects.size(); ++r)
          if (p.rects[r].group == (int)g) { G.rects.push_back((int)r); mx = std::max(mx, p.rects[r].ws_bytes); }
        G.arena_bytes = align_up(mx, WS_ALIGN);
        off += G.arena_bytes;
        p.groups.push_back(G);
      }
      p.ws_bytes = off;
      set_error("");
      return TLR_OK;
    }
    regs = make_regions(p, false);   // fall back to one sequential region
  }
  std::vector<Rect> rr;
  tlr_status st = schedule_region(p, s, regs[0], budget, 0, rr);
  if (st != TLR_OK) return st;
  p.rects = rr;
  Group G;
  G.stream = 0;
  G.arena_off = 0;
  size_t mx = 0;
  for (size_t r = 0; r < p.rects.size(); ++r) { G.rects.push_back((int)r); mx = std::max(mx, p.rects[r].ws_bytes); }
  G.arena_bytes = align_up(mx, WS_ALIGN);
  p.groups.push_back(G);
  p.ws_bytes = G.arena_bytes;
  return TLR_OK;
}

// ---------------------------------------------------------------------------
// Descriptor generation.

static DevOperand opnd(uint8_t base, int64_t off, int64_t ld, int trans) {
  DevOperand o;
  o.off = off;
  o.ld = (int32_t)ld;
  o.base = base;
  o.trans = (uint8_t)trans;
  o.flags = 0;
  return o;
}

// a workspace operand allocated with whole ld-strided vectors: padded when ld
// exceeds its extent along the contiguous index
static DevOperand padded(DevOperand o, int64_t extent) {
  if (o.ld > extent) o.flags |= OPND_PADDED;
  return o;
}

struct TaskList {
  std::vector<DevTask> t;
  std::vector<double> useful;  // per task
};

static DevTask new_task(int64_t M, int64_t N, uint8_t cbase, int64_t c_off, int64_t ldc,
                        int64_t ctab, bool final_) {
  DevTask d;
  std::memset(&d, 0, sizeof(d));
  d.M = (int32_t)M;
  d.N = (int32_t)N;
  d.c_off = c_off;
  d.ctab = ctab;
  d.ldc = (int32_t)ldc;
  d.c_base = cbase;
  d.final_ = final_ ? 1 : 0;
  d.nseg = 0;
  return d;
}

static void add_seg(DevTask &d, DevOperand a, DevOperand b, int64_t K) {
  if (K <= 0) return;
  DevSeg &s = d.seg[d.nseg++];
  s.a = a;
  s.b = b;
  s.K = (int32_t)K;
  s.pad = 0;
}

static double task_exec_flops(const DevTask &d) {
  double F = 0;
  for (int s = 0; s < d.nseg; ++s) F += 2.0 * d.M * (double)d.N * d.seg[s].K;
  return F;
}

// Emit the workgroup table of one launch: one sub-table per load mode of the
// tasks (tlr_desc.h), each built the same way.  Workgroups are dealt to the 8
// XCDs round-robin by index (index x, x+8, x+16, ... run on XCD x, each XCD in
// its own order), so a sub-table is built per XCD: whole tasks (all blocks of
// one output tile stay on one XCD and share its L2) go, longest first, to the
// XCD with the least work so far, and each XCD's list runs longest first.
// Lists are padded with idle entries to a common length, so every sub-table
// is a multiple of NUM_XCD entries and the XCD of an entry does not depend on
// which sub-tables precede it.
// Block width of a launch.  128 x 128 blocks move the fewest operand bytes per
// flop; 128 x 64 blocks (half the accumulators, four workgroups per CU) spread
// a launch of few blocks over more CUs.  The final update stays wide; the
// others go narrow when 128 x 128 blocks would give fewer than four workgroups
// per CU (the coupling and diagonal-term GEMMs: few, with K = b).  Measured on
// the store-bound right/left product, narrow blocks were no faster.
// 16-bit launches whose 256 x 256 blocks still fill the chip twice take them
// (the final update always): a 128 x 128 block of the store-bound
// right/left product writes only 32 KB and spends most of its time on the
// fixed cost of a block.  Measured on N = 32768 (heavy ranks): right/left
// product 1.22 -> 1.10 ms, coupling 0.44 -> 0.39 ms; launches of fewer
// wide blocks (the couplings at N = 16384) ran slower in them.
static bool wide16(int stage, const TaskList &tl) {
  if (stage == 3) return true;
  int64_t blocks = 0;
  for (const DevTask &d : tl.t) blocks += ceil_div(d.M, BW16) * ceil_div(d.N, BW16);
  return blocks >= 2 * 256;
}

static int launch_bn(int stage, const TaskList &tl) {
  if (stage == 3) return BN;
  int64_t blocks = 0;
  for (const DevTask &d : tl.t) blocks += ceil_div(d.M, BM) * ceil_div(d.N, BN);
  return blocks < 4 * 256 ? BN_NARROW : BN;
}

// A right/left-product task that the strip kernel runs: at most one K segment
// of at most STRIP_K, B N-contiguous, output C = acc (32/64-bit types); on
// 16-bit types at most STRIP_K16, either layout of A and B.
static bool strip_task(const Plan &p, const DevTask &d) {
  if (d.final_ || d.nseg > 1) return false;
  if (d.nseg == 0) return true;
  if (p.es == 2) return d.seg[0].K <= STRIP_K16;
  return d.seg[0].K <= STRIP_K && d.seg[0].b.trans == 1;
}

// Appends one launch of `tl` (nothing when empty) and returns its index, or -1.
// A strip launch takes 128 x STRIP_W blocks.
static int emit_launch(Plan &p, int stage, int group, int rect, TaskList &tl, bool strip = false) {
  if (tl.t.empty()) return -1;
  Launch L;
  L.stage = stage;
  L.group = group;
  L.rect = rect;
  L.wait_launch = -1;
  L.fork_at = -1;
  L.on_side = false;
  L.beta_one = false;
  L.n_tasks = (int64_t)tl.t.size();
  L.useful_flops = 0;
  L.executed_flops = 0;
  const int32_t task0 = (int32_t)p.tasks.size();
  L.task_off = task0;
  L.bn = strip ? STRIP_W : launch_bn(stage, tl);
  L.bm = BM;
  if (p.es == 2 && !strip && wide16(stage, tl)) L.bm = L.bn = BW16;   // 16-bit: 256 x 256 blocks
  const int bm = L.bm, bn = L.bn;
  struct TaskCost { int32_t t; int64_t per_block, blocks; int mode; };
  std::vector<TaskCost> order;
  for (size_t t = 0; t < tl.t.size(); ++t) {
    const DevTask &d = tl.t[t];
    L.useful_flops += tl.useful[t];
    L.executed_flops += task_exec_flops(d);
    int64_t K = 0;
    for (int s = 0; s < d.nseg; ++s) K += d.seg[s].K;
    const int64_t blocks = ceil_div(d.M, bm) * ceil_div(d.N, bn);
    // one block costs its K steps plus a fixed share for the C update
    order.push_back({(int32_t)t, K + 32, blocks, task_load_mode(d)});
    p.tasks.push_back(d);
  }
  std::stable_sort(order.begin(), order.end(),
                   [](const TaskCost &a, const TaskCost &b) { return a.per_block > b.per_block; });
  L.tile_off = (int64_t)p.tiles.size();
  for (int mode = 0; mode < NUM_LOAD_MODES; ++mode) {
    std::vector<std::vector<DevTile>> xl(NUM_XCD);
    std::vector<int64_t> load(NUM_XCD, 0);
    for (const TaskCost &c : order) {
      if (c.mode != mode) continue;
      int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      load[x] += c.per_block * c.blocks;
      const DevTask &d = tl.t[c.t];
      for (int64_t m0 = 0; m0 < d.M; m0 += bm)
        for (int64_t n0 = 0; n0 < d.N; n0 += bn)
          xl[x].push_back(DevTile{task0 + c.t, (int32_t)m0, (int32_t)n0, 0});
    }
    size_t per = 0;
    for (auto &v : xl) per = std::max(per, v.size());
    std::vector<DevTile> tab(per * NUM_XCD, DevTile{-1, 0, 0, 0});
    for (int x = 0; x < NUM_XCD; ++x)
      for (size_t t = 0; t < xl[x].size(); ++t) tab[t * NUM_XCD + x] = xl[x][t];
    L.mode_off[mode] = (int64_t)p.tiles.size() - L.tile_off;
    L.mode_tiles[mode] = (int64_t)tab.size();
    p.tiles.insert(p.tiles.end(), tab.begin(), tab.end());
  }
  L.n_tiles = (int64_t)p.tiles.size() - L.tile_off;
  p.launches.push_back(L);
  p.groups[group].launches.push_back((int)p.launches.size() - 1);
  return (int)p.launches.size() - 1;
}

// Launches of one rectangle: the coupling (stage 1), then the diagonal-term
// products that read only inputs on the side stream (forked before stage 1, so
// they run beside stages 1 and 2), the right/left product (stage 2) and the
// final update (stage 3), which waits for the side launch.
// The right/left product is split: tasks with K <= STRIP_K (16-bit types:
// STRIP_K16) go to a strip launch on the group's stream, the rest to a
// grouped launch on the side stream (below).  The split is made only when the strip launch
// would fill the chip twice (STRIP_MIN_BLOCKS workgroups); a handful of strip
// tasks beside the grouped launch measured slower than leaving them in it.
constexpr int64_t STRIP_MIN_BLOCKS = 2 * 256;
static void emit_stages(Plan &p, int group, int rect, TaskList &l1, TaskList &side, TaskList &l2,
                        TaskList &l3) {
  const int a = emit_launch(p, 1, group, rect, l1);
  const int d = emit_launch(p, STAGE_SIDE, group, rect, side);
  TaskList l2s, l2g;
  int64_t strip_blocks = 0;
  for (size_t t = 0; t < l2.t.size(); ++t) {
    const DevTask &x = l2.t[t];
    const bool s = strip_task(p, x);
    if (s) strip_blocks += ceil_div(x.M, BM) * ceil_div(x.N, STRIP_W);
    TaskList &dst = s ? l2s : l2g;
    dst.t.push_back(x);
    dst.useful.push_back(l2.useful[t]);
  }
  if (strip_blocks < STRIP_MIN_BLOCKS) {
    l2g = l2;
    l2s = TaskList();
  }
  // Beside a strip launch the grouped one goes to the side stream, after the
  // side launch, waiting for the coupling: its MFMA-heavy blocks then run
  // beside the strip launch's stores instead of before them.  (Waiting for
  // the coupling also orders it after everything the group's stream held
  // before, the previous rectangle's final update included.)
  const bool split = !l2s.t.empty() && !l2g.t.empty() && a >= 0;
  const int g2 = emit_launch(p, 2, group, rect, l2g);
  if (split) {
    p.launches[g2].on_side = true;
    p.launches[g2].wait_launch = a;
  }
  emit_launch(p, 2, group, rect, l2s, true);
  const int c = emit_launch(p, 3, group, rect, l3);
  if (split && c >= 0) p.launches[c].wait_launch = g2;   // the side stream holds the side launch before it
  if (d < 0) return;
  // fork before the coupling launch, so that the side launch runs beside
  // stages 1 and 2.  Without a coupling launch the fork is the side launch's
  // own position (fork_at -1): its event is then recorded on the group's
  // stream after everything enqueued there so far and before the side stream
  // waits on it.  A later launch (stage 2 or 3) would record the event only
  // after the side stream's wait has been enqueued, which orders nothing.
  p.launches[d].fork_at = a;
  if (c >= 0 && !split) p.launches[c].wait_launch = d;
}

static void emit_rect(Plan &p, const Sums &s, int rect) {
  const Rect &R = p.rects[rect];
  const View &A = p.A;
  const View &B = p.B;
  const int64_t es = p.es;
  const int64_t b = A.b;
  const int i0 = R.i0, i1 = R.i1, j0 = R.j0, j1 = R.j1;
  const int64_t WJ = width(p, j0, j1), WI = height(p, i0, i1);
  const size_t arena = p.groups[R.group].arena_off;
  size_t cur = arena;
  auto take = [&](size_t bytes) {
    int64_t off = (int64_t)(cur / (size_t)es);
    cur += align_up(bytes, WS_ALIGN);
    return off;
  };
  const int qk = s.qk;
  // column offset of tile j inside the J block / row offset of tile i inside I
  auto cJ = [&](int j) { return p.no[j] - p.no[j0]; };
  auto rI = [&](int i) { return A.ro[i] - A.ro[i0]; };

  if (p.dense_b) {
    std::vector<int64_t> Toff(s.qm, -1);
    for (int i = i0; i < i1; ++i)
      if (s.rho[i] > 0) Toff[i] = take((size_t)WJ * s.rho[i] * es);
    // launch 1: T_i^T[n, p_i(k)+a] = sum_kk op(B)[k rows, J cols]^T V_ik
    TaskList l1;
    const int64_t c0 = p.no[j0];
    for (int k = 0; k < qk; ++k) {
      int64_t kap = s.kap(k, i0, i1);
      if (kap == 0) continue;
      int64_t ctab = (int64_t)p.coltab.size();
      for (int i = i0; i < i1; ++i) {
        int64_t pik = 0;
        for (int kk = 0; kk < k; ++kk) pik += A.r(i, kk);
        for (int a = 0; a < A.r(i, k); ++a) p.coltab.push_back(Toff[i] + (pik + a) * WJ);
      }
      DevTask d = new_task(WJ, kap, BASE_WS, 0, 0, ctab, false);
      DevOperand ao = p.opB == TLR_OP_N ? opnd(BASE_B_DENSE, A.co[k] + c0 * p.ldb, p.ldb, 1)
                                        : opnd(BASE_B_DENSE, c0 + A.co[k] * p.ldb, p.ldb, 0);
      add_seg(d, ao, opnd(A.inner_base, A.ic(i0, k) * b, b, 0), A.cs[k]);
      l1.t.push_back(d);
      l1.useful.push_back(2.0 * WJ * A.cs[k] * kap);
    }
    emit_launch(p, 1, R.group, rect, l1);
    TaskList l3;
    for (int i = i0; i < i1; ++i)
      for (int j = j0; j < j1; ++j) {
        DevTask d = new_task(A.rs[i], p.ns[j], BASE_C, A.ro[i] + p.no[j] * p.ldc, p.ldc, -1, true);
        double u = 0;
        if (s.rho[i] > 0) {
          add_seg(d, opnd(A.outer_base, A.oc(i, 0) * b, b, 0), opnd(BASE_WS, Toff[i] + cJ(j), WJ, 1), s.rho[i]);
          u += 2.0 * A.rs[i] * (double)p.ns[j] * s.rho[i];
        }
        if (A.diag) {
          DevOperand bo = p.opB == TLR_OP_N ? opnd(BASE_B_DENSE, A.ro[i] + p.no[j] * p.ldb, p.ldb, 0)
                                            : opnd(BASE_B_DENSE, p.no[j] + A.ro[i] * p.ldb, p.ldb, 1);
          add_seg(d, opnd(A.diag_base, (int64_t)i * b * b, b, A.diag_trans), bo, A.rs[i]);
          u += 2.0 * A.rs[i] * (double)A.rs[i] * p.ns[j];
        }
        l3.t.push_back(d);
        l3.useful.push_back(u);
      }
    emit_launch(p, 3, R.group, rect, l3);
    return;
  }

  if (p.dense_a) {
    // dense A: the left order with the coupling replaced by the product itself
    // (launch 1: Y_j[:, (k, a)] = op(A)[I rows, k-block] W_kj[:, a] through a
    // column map), then Y_j Z_j^T plus op(A)[i rows, j-block] op(D_B,jj)
    const int64_t lda = p.ldb;
    auto a_block = [&](int64_t r0, int64_t c0) {   // op(A)[r0.., c0..] as an M x K operand
      return p.opA == TLR_OP_N ? opnd(BASE_B_DENSE, r0 + c0 * lda, lda, 0) : opnd(BASE_B_DENSE, c0 + r0 * lda, lda, 1);
    };
    std::vector<int64_t> Yoff(s.qn, -1);
    for (int j = j0; j < j1; ++j)
      if (s.gam[j] > 0) Yoff[j] = take((size_t)WI * s.gam[j] * es);
    TaskList l1, l3;
    for (int k = 0; k < qk; ++k) {
      const int64_t SN = s.bet(k, j0, j1);
      if (SN == 0) continue;
      const int64_t ctab = (int64_t)p.coltab.size();
      for (int j = j0; j < j1; ++j) {
        int64_t pkj = 0;
        for (int kk = 0; kk < k; ++kk) pkj += B.r(kk, j);
        for (int a = 0; a < B.r(k, j); ++a) p.coltab.push_back(Yoff[j] + (pkj + a) * WI);
      }
      DevTask d = new_task(WI, SN, BASE_WS, 0, 0, ctab, false);
      add_seg(d, a_block(A.ro[i0], A.co[k]), opnd(B.outer_base, B.oc(k, j0) * b, b, 0), A.cs[k]);
      l1.t.push_back(d);
      l1.useful.push_back(2.0 * WI * (double)SN * A.cs[k]);
    }
    for (int j = j0; j < j1; ++j)
      for (int i = i0; i < i1; ++i) {
        DevTask d = new_task(A.rs[i], p.ns[j], BASE_C, A.ro[i] + p.no[j] * p.ldc, p.ldc, -1, true);
        double u = 0;
        if (s.gam[j] > 0) {
          add_seg(d, opnd(BASE_WS, Yoff[j] + rI(i), WI, 0), opnd(B.inner_base, B.ic(0, j) * b, b, 1), s.gam[j]);
          u += 2.0 * A.rs[i] * (double)p.ns[j] * s.gam[j];
        }
        if (B.diag) {
          add_seg(d, a_block(A.ro[i], A.co[j]), opnd(B.diag_base, (int64_t)j * b * b, b, B.diag_trans), p.ns[j]);
          u += 2.0 * A.rs[i] * (double)p.ns[j] * p.ns[j];
        }
        l3.t.push_back(d);
        l3.useful.push_back(u);
      }
    emit_launch(p, 1, R.group, rect, l1);
    emit_launch(p, 3, R.group, rect, l3);
    return;
  }

  // coupling blocks S_k (kap_k(I) x bet_k(J), column-major)
  std::vector<int64_t> Soff(qk, -1), SM(qk, 0), SN(qk, 0);
  for (int k = 0; k < qk; ++k) {
    SM[k] = s.kap(k, i0, i1);
    SN[k] = s.bet(k, j0, j1);
    if (SM[k] > 0 && SN[k] > 0) Soff[k] = take((size_t)s_elems(SM[k], SN[k], R.order) * es);
  }
  TaskList l1, ls, l2, l3;
  for (int k = 0; k < qk; ++k) {
    if (Soff[k] < 0) continue;
    const int64_t ls = s_ld(SM[k], SN[k], R.order);
    if (R.order == TLR_ORDER_RIGHT) {
      // S_k = V_{I,k}^T W_{k,J}
      DevTask d = new_task(SM[k], SN[k], BASE_WS, Soff[k], ls, -1, false);
      add_seg(d, opnd(A.inner_base, A.ic(i0, k) * b, b, 1), opnd(B.outer_base, B.oc(k, j0) * b, b, 0), A.cs[k]);
      l1.t.push_back(d);
    } else {
      // S_k^T = W_{k,J}^T V_{I,k}
      DevTask d = new_task(SN[k], SM[k], BASE_WS, Soff[k], ls, -1, false);
      add_seg(d, opnd(B.outer_base, B.oc(k, j0) * b, b, 1), opnd(A.inner_base, A.ic(i0, k) * b, b, 0), A.cs[k]);
      l1.t.push_back(d);
    }
    l1.useful.push_back(2.0 * SM[k] * (double)SN[k] * A.cs[k]);
  }

  if (R.order == TLR_ORDER_RIGHT) {
    std::vector<int64_t> Toff(s.qm, -1), Xoff(s.qm, -1);
    for (int i = i0; i < i1; ++i) {
      if (s.rho[i] > 0) Toff[i] = take((size_t)WJ * s.rho[i] * es);
      if (A.diag && s.bet(i, j0, j1) > 0) Xoff[i] = take((size_t)A.rs[i] * s.bet(i, j0, j1) * es);
    }
    // X_i = op(D_A,ii) W_{i,J} (inputs only: side launch)
    if (A.diag)
      for (int i = i0; i < i1; ++i) {
        int64_t bi = s.bet(i, j0, j1);
        if (bi == 0) continue;
        DevTask d = new_task(A.rs[i], bi, BASE_WS, Xoff[i], A.rs[i], -1, false);
        add_seg(d, opnd(A.diag_base, (int64_t)i * b * b, b, A.diag_trans), opnd(B.outer_base, B.oc(i, j0) * b, b, 0), A.rs[i]);
        ls.t.push_back(d);
        ls.useful.push_back(2.0 * A.rs[i] * (double)A.rs[i] * bi);
      }
    // column maps: coupling row (i, a) of contraction tile k -> column p_i(k)+a of T_i^T
    std::vector<int64_t> ctab(qk, -1);
    for (int k = 0; k < qk; ++k) {
      if (SM[k] == 0) continue;
      ctab[k] = (int64_t)p.coltab.size();
      for (int i = i0; i < i1; ++i) {
        int64_t pik = 0;
        for (int kk = 0; kk < k; ++kk) pik += A.r(i, kk);
        for (int a = 0; a < A.r(i, k); ++a) p.coltab.push_back(Toff[i] + (pik + a) * WJ);
      }
    }
    for (int k = 0; k < qk; ++k) {
      if (SM[k] == 0) continue;
      int64_t boff = 0;   // column offset of block j inside S_k
      for (int j = j0; j < j1; ++j) {
        DevTask d = new_task(p.ns[j], SM[k], BASE_WS, cJ(j), 0, ctab[k], false);
        if (B.diag && k == j) {
          // T_i[j-block rows, j-block cols] = V_ij^T D_B,jj, stored transposed:
          // D^T V (inputs only: side launch)
          add_seg(d, opnd(B.diag_base, (int64_t)j * b * b, b, B.diag_trans ? 0 : 1),
                  opnd(A.inner_base, A.ic(i0, j) * b, b, 0), p.ns[j]);
          ls.t.push_back(d);
          ls.useful.push_back(2.0 * p.ns[j] * (double)p.ns[j] * SM[k]);
          continue;
        }
        const int32_t r = B.r(k, j);
        if (r > 0)
          add_seg(d, opnd(B.inner_base, B.ic(k, j) * b, b, 0),
                  padded(opnd(BASE_WS, Soff[k] + boff * s_ld(SM[k], SN[k], R.order), s_ld(SM[k], SN[k], R.order), 1), SM[k]), r);
        boff += r;
        l2.t.push_back(d);
        l2.useful.push_back(2.0 * p.ns[j] * (double)SM[k] * r);   // r == 0 writes a zero block
      }
    }
    for (int i = i0; i < i1; ++i) {
      for (int j = j0; j < j1; ++j) {
        DevTask d = new_task(A.rs[i], p.ns[j], BASE_C, A.ro[i] + p.no[j] * p.ldc, p.ldc, -1, true);
        int64_t kk = 0;
        for (int k = 0; k < qk; ++k)
          if (B.r(k, j) > 0 || (B.diag && k == j)) kk += A.r(i, k);
        double u = 2.0 * A.rs[i] * (double)p.ns[j] * kk;
        if (s.rho[i] > 0)
          add_seg(d, opnd(A.outer_base, A.oc(i, 0) * b, b, 0), opnd(BASE_WS, Toff[i] + cJ(j), WJ, 1), s.rho[i]);
        if (A.diag) {
          if (B.diag && i == j) {
            add_seg(d, opnd(A.diag_base, (int64_t)i * b * b, b, A.diag_trans),
                    opnd(B.diag_base, (int64_t)i * b * b, b, B.diag_trans), A.rs[i]);
            u += 2.0 * A.rs[i] * (double)A.rs[i] * A.rs[i];
          } else if (B.r(i, j) > 0) {
            int64_t xo = s.bet(i, j0, j);
            add_seg(d, opnd(BASE_WS, Xoff[i] + xo * A.rs[i], A.rs[i], 0),
                    opnd(B.inner_base, B.ic(i, j) * b, b, 1), B.r(i, j));
            u += 2.0 * A.rs[i] * (double)p.ns[j] * B.r(i, j);
          }
        }
        l3.t.push_back(d);
        l3.useful.push_back(u);
      }
    }
  } else {
    std::vector<int64_t> Yoff(s.qn, -1), Xoff(s.qn, -1);
    for (int j = j0; j < j1; ++j) {
      if (s.gam[j] > 0) Yoff[j] = take((size_t)WI * s.gam[j] * es);
      if (B.diag && s.kap(j, i0, i1) > 0) Xoff[j] = take((size_t)s.kap(j, i0, i1) * p.ns[j] * es);
    }
    // X'_j = V_{I,j}^T op(D_B,jj) (inputs only: side launch)
    if (B.diag)
      for (int j = j0; j < j1; ++j) {
        int64_t kj = s.kap(j, i0, i1);
        if (kj == 0) continue;
        DevTask d = new_task(kj, p.ns[j], BASE_WS, Xoff[j], kj, -1, false);
        add_seg(d, opnd(A.inner_base, A.ic(i0, j) * b, b, 1), opnd(B.diag_base, (int64_t)j * b * b, b, B.diag_trans), p.ns[j]);
        ls.t.push_back(d);
        ls.useful.push_back(2.0 * kj * (double)p.ns[j] * p.ns[j]);
      }
    // column maps: coupling column (j, a) of contraction tile k -> column p'_j(k)+a of Y_j
    std::vector<int64_t> ytab(qk, -1);
    for (int k = 0; k < qk; ++k) {
      if (SN[k] == 0) continue;
      ytab[k] = (int64_t)p.coltab.size();
      for (int j = j0; j < j1; ++j) {
        int64_t pkj = 0;
        for (int kk = 0; kk < k; ++kk) pkj += B.r(kk, j);
        for (int a = 0; a < B.r(k, j); ++a) p.coltab.push_back(Yoff[j] + (pkj + a) * WI);
      }
    }
    for (int i = i0; i < i1; ++i) {
      for (int k = 0; k < qk; ++k) {
        if (SN[k] == 0) continue;
        DevTask d = new_task(A.rs[i], SN[k], BASE_WS, rI(i), 0, ytab[k], false);
        if (A.diag && k == i) {
          // Y_j[i rows, k = i block] = op(D_A,ii) W_ij (inputs only: side launch)
          add_seg(d, opnd(A.diag_base, (int64_t)i * b * b, b, A.diag_trans), opnd(B.outer_base, B.oc(i, j0) * b, b, 0), A.rs[i]);
          ls.t.push_back(d);
          ls.useful.push_back(2.0 * A.rs[i] * (double)A.rs[i] * SN[k]);
          continue;
        }
        const int32_t r = A.r(i, k);
        if (r > 0) {
          const int64_t ao = s.kap(k, i0, i);
          // rows ao.. of S_k, read from S_k^T: N (beta) contiguous
          const int64_t lt = s_ld(SM[k], SN[k], R.order);
          add_seg(d, opnd(A.outer_base, A.oc(i, k) * b, b, 0), padded(opnd(BASE_WS, Soff[k] + ao * lt, lt, 1), SN[k]), r);
        }
        l2.t.push_back(d);
        l2.useful.push_back(2.0 * A.rs[i] * (double)SN[k] * r);
      }
    }
    for (int j = j0; j < j1; ++j) {
      for (int i = i0; i < i1; ++i) {
        DevTask d = new_task(A.rs[i], p.ns[j], BASE_C, A.ro[i] + p.no[j] * p.ldc, p.ldc, -1, true);
        int64_t kk = 0;
        for (int k = 0; k < qk; ++k)
          if (A.r(i, k) > 0 || (A.diag && k == i)) kk += B.r(k, j);
        double u = 2.0 * A.rs[i] * (double)p.ns[j] * kk;
        if (s.gam[j] > 0)
          add_seg(d, opnd(BASE_WS, Yoff[j] + rI(i), WI, 0), opnd(B.inner_base, B.ic(0, j) * b, b, 1), s.gam[j]);
        if (B.diag) {
          if (A.diag && i == j) {
            add_seg(d, opnd(A.diag_base, (int64_t)i * b * b, b, A.diag_trans),
                    opnd(B.diag_base, (int64_t)i * b * b, b, B.diag_trans), A.rs[i]);
            u += 2.0 * A.rs[i] * (double)A.rs[i] * A.rs[i];
          } else if (A.r(i, j) > 0) {
            int64_t ao = s.kap(j, i0, i);
            add_seg(d, opnd(A.outer_base, A.oc(i, j) * b, b, 0), opnd(BASE_WS, Xoff[j] + ao, s.kap(j, i0, i1), 0), A.r(i, j));
            u += 2.0 * A.rs[i] * (double)p.ns[j] * A.r(i, j);
          }
        }
        l3.t.push_back(d);
        l3.useful.push_back(u);
      }
    }
  }
  emit_stages(p, R.group, rect, l1, ls, l2, l3);
}

static double compressed_elems(const View &v) {
  double e = 0;
  for (int i = 0; i < v.qr; ++i)
    for (int j = 0; j < v.qc; ++j) {
      if (v.diag && i == j) e += (double)v.rs[i] * v.rs[i];
      else e += (double)v.r(i, j) * (v.rs[i] + v.cs[j]);
    }
  return e;
}

// ---------------------------------------------------------------------------
// Descriptor self-check.  Always: every element a task's operands or output can
// touch lies inside its buffer, and every workgroup table covers each block of
// each task exactly once.  With TLR_PLAN_VALIDATE also: writes inside one launch
// never overlap, every workspace element a launch reads was written by an
// earlier launch of the same rectangle, and every element of C is written once.

struct BufSizes {
  int64_t n[NUM_BASES];
};

static int64_t view_factor_elems(const View &v) {
  int64_t s = 0;
  for (int32_t r : v.R) s += r;
  return s * v.b;
}

static BufSizes buffer_sizes(const Plan &p) {
  BufSizes z;
  for (auto &x : z.n) x = 0;
  z.n[BASE_A_OUTER] = z.n[BASE_A_INNER] = view_factor_elems(p.A);
  z.n[BASE_A_DIAG] = p.A.diag ? (int64_t)p.A.qr * p.A.b * p.A.b : 0;
  if (!p.dense_b) {
    z.n[BASE_B_OUTER] = z.n[BASE_B_INNER] = view_factor_elems(p.B);
    z.n[BASE_B_DIAG] = p.B.diag ? (int64_t)p.B.qr * p.B.b * p.B.b : 0;
  }
  if ((p.dense_b || p.dense_a) && p.dense_cols > 0 && p.dense_rows > 0)   // the dense operand, A or B
    z.n[BASE_B_DENSE] = p.ldb * (p.dense_cols - 1) + p.dense_rows;
  z.n[BASE_WS] = (int64_t)(p.ws_bytes / (size_t)p.es);
  if (p.m > 0 && p.n > 0) z.n[BASE_C] = p.ldc * (p.n - 1) + p.m;
  return z;
}

static bool operand_ok(const DevOperand &o, int64_t rows, int64_t cols, bool is_a, const BufSizes &z) {
  // is_a: (rows, cols) = (M, K); else (K, N).  trans picks which index is contiguous.
  // the kernel forms intra-tile byte offsets up to (127*ld + 15)*8, below 2^31
  if (o.base >= NUM_BASES || o.off < 0 || o.ld < 1 || o.ld >= (1 << 21)) return false;
  if (rows == 0 || cols == 0) return true;
  const bool first_contig = (o.trans == 0);   // A: M contiguous / B: K contiguous
  int64_t a = first_contig ? rows : cols, c = first_contig ? cols : rows;
  (void)is_a;
  int64_t last = o.off + (a - 1) + (c - 1) * (int64_t)o.ld;
  // a padded operand claims whole ld-strided vectors (and the pair loads use it)
  if (o.flags & OPND_PADDED) {
    if (o.ld <= a) return false;
    last = o.off + c * (int64_t)o.ld - 1;
  }
  return last < z.n[o.base];
}

static tlr_status validate(const Plan &p, bool deep) {
  const BufSizes z = buffer_sizes(p);
  for (size_t t = 0; t < p.tasks.size(); ++t) {
    const DevTask &d = p.tasks[t];
    if (d.M < 0 || d.N < 0 || d.nseg > 2) return fail(TLR_ERR_INVALID_ARG, "internal: malformed task");
    for (int s = 0; s < d.nseg; ++s) {
      if (d.seg[s].K <= 0) return fail(TLR_ERR_INVALID_ARG, "internal: empty segment");
      if (!operand_ok(d.seg[s].a, d.M, d.seg[s].K, true, z) || !operand_ok(d.seg[s].b, d.seg[s].K, d.N, false, z))
        return fail(TLR_ERR_INVALID_ARG, "internal: operand range outside its buffer (task " + std::to_string(t) + ")");
    }
    if (d.M == 0 || d.N == 0) continue;
    if (d.c_base >= NUM_BASES || d.c_off < 0) return fail(TLR_ERR_INVALID_ARG, "internal: bad output");
    int64_t lo, hi;
    if (d.ctab < 0) {
      if (d.ldc < d.M) return fail(TLR_ERR_INVALID_ARG, "internal: output columns overlap");
      lo = d.c_off;
      hi = d.c_off + (d.M - 1) + (int64_t)(d.N - 1) * d.ldc;
    } else {
      if (d.ctab + d.N > (int64_t)p.coltab.size()) return fail(TLR_ERR_INVALID_ARG, "internal: column map overrun");
      lo = std::numeric_limits<int64_t>::max();
      hi = -1;
      for (int n = 0; n < d.N; ++n) {
        lo = std::min(lo, d.c_off + p.coltab[d.ctab + n]);
        hi = std::max(hi, d.c_off + p.coltab[d.ctab + n] + d.M - 1);
      }
    }
    if (lo < 0 || hi >= z.n[d.c_base])
      return fail(TLR_ERR_INVALID_ARG, "internal: output range outside its buffer (task " + std::to_string(t) + ")");
  }
  // workgroup tables: each block of each task exactly once
  std::vector<int64_t> seen(p.tasks.size(), 0), want(p.tasks.size(), -1);
  for (const Launch &L : p.launches) {
    const bool strip = L.bm == BM && L.bn == STRIP_W;
    const bool shape_ok = strip ? L.stage == 2
                          : L.bm == BM ? (L.bn == BN || L.bn == BN_NARROW)
                                       : (L.bm == BW16 && L.bn == BW16 && p.es == 2);
    if (!shape_ok || L.task_off < 0 || L.task_off + L.n_tasks > (int64_t)p.tasks.size())
      return fail(TLR_ERR_INVALID_ARG, "internal: bad launch block shape or task range");
    for (int64_t t = L.task_off; t < L.task_off + L.n_tasks; ++t) {
      // the strip kernel holds one K stage and fills LDS from an N-contiguous B
      if (strip && !strip_task(p, p.tasks[t]))
        return fail(TLR_ERR_INVALID_ARG, "internal: task in a strip launch that the strip kernel cannot run");
      want[t] = ceil_div(p.tasks[t].M, L.bm) * ceil_div(p.tasks[t].N, L.bn);
    }
  }
  for (const Launch &L : p.launches) {
    if (L.tile_off < 0 || L.tile_off + L.n_tiles > (int64_t)p.tiles.size() || L.n_tiles % NUM_XCD)
      return fail(TLR_ERR_INVALID_ARG, "internal: launch table out of range");
    // the per-mode sub-tables tile the launch's table, and a pair mode only
    // holds tasks that qualify for it: its loads rely on that for staying
    // inside the operands
    int64_t covered = 0;
    for (int m = 0; m < NUM_LOAD_MODES; ++m) {
      if (L.mode_off[m] != covered || L.mode_tiles[m] < 0 || L.mode_tiles[m] % NUM_XCD)
        return fail(TLR_ERR_INVALID_ARG, "internal: load-mode tables malformed");
      covered += L.mode_tiles[m];
    }
    if (covered != L.n_tiles) return fail(TLR_ERR_INVALID_ARG, "internal: load-mode tables malformed");
    for (int64_t e = L.tile_off; e < L.tile_off + L.n_tiles; ++e) {
      const DevTile &x = p.tiles[e];
      if (x.task < 0) continue;
      if (x.task >= (int32_t)p.tasks.size()) return fail(TLR_ERR_INVALID_ARG, "internal: bad task index");
      const DevTask &d = p.tasks[x.task];
      int mode = 0;
      while (mode + 1 < NUM_LOAD_MODES && e >= L.tile_off + L.mode_off[mode + 1]) ++mode;
      if (mode != LOAD_SINGLE && task_load_mode(d) != mode)
        return fail(TLR_ERR_INVALID_ARG, "internal: task in the table of a load mode it does not qualify for");
      if (x.task < L.task_off || x.task >= L.task_off + L.n_tasks)
        return fail(TLR_ERR_INVALID_ARG, "internal: workgroup entry of another launch's task");
      if (x.m0 < 0 || x.n0 < 0 || x.m0 >= d.M || x.n0 >= d.N || x.m0 % L.bm || x.n0 % L.bn)
        return fail(TLR_ERR_INVALID_ARG, "internal: bad block origin");
      seen[x.task]++;
    }
  }
  for (size_t t = 0; t < p.tasks.size(); ++t)
    if (seen[t] != want[t]) return fail(TLR_ERR_INVALID_ARG, "internal: blocks of a task missing or repeated");
  // stream order: the executor enqueues the groups one after another, each
  // group's launches in list order.  An event must be recorded before a
  // stream waits on it in the same execute, otherwise the wait sees the
  // previous execute's record (or none) and orders nothing.  So a side
  // launch's fork point (where its fork event is recorded on the group's
  // stream) is in its own group at or before it, and a launch waits only for
  // a launch enqueued earlier.
  {
    std::vector<int64_t> pos(p.launches.size(), -1);
    std::vector<int> grp(p.launches.size(), -1);
    int64_t at = 0;
    for (size_t g = 0; g < p.groups.size(); ++g)
      for (int l : p.groups[g].launches) {
        if (l < 0 || l >= (int)p.launches.size() || pos[l] >= 0)
          return fail(TLR_ERR_INVALID_ARG, "internal: launch lists of the groups malformed");
        pos[l] = at++;
        grp[l] = (int)g;
      }
    for (size_t l = 0; l < p.launches.size(); ++l) {
      const Launch &L = p.launches[l];
      if (pos[l] < 0) return fail(TLR_ERR_INVALID_ARG, "internal: launch in no group");
      if (L.stage == STAGE_SIDE && L.fork_at >= 0) {
        if (L.fork_at >= (int)p.launches.size() || grp[L.fork_at] != grp[l] || pos[L.fork_at] > pos[l])
          return fail(TLR_ERR_INVALID_ARG, "internal: side launch " + std::to_string(l) +
                                               " forks after its own wait is enqueued");
      }
      if (L.wait_launch >= 0) {
        if (L.wait_launch >= (int)p.launches.size() || pos[L.wait_launch] >= pos[l])
          return fail(TLR_ERR_INVALID_ARG, "internal: launch " + std::to_string(l) +
                                               " waits for a launch enqueued after it");
      }
    }
  }
  if (!deep) return TLR_OK;

  // deep check: replay every launch on per-element state
  std::vector<uint8_t> ws((size_t)z.n[BASE_WS], 0);
  std::vector<uint64_t> cbits((size_t)((z.n[BASE_C] + 63) / 64), 0);
  int64_t cwrites = 0;
  const bool per_k = (p.flags & TLR_PLAN_PER_K) != 0;
  auto for_elems = [&](const DevOperand &o, int64_t rows, int64_t cols, auto &&fn) {
    const bool fc = o.trans == 0;
    const int64_t a = fc ? rows : cols, c = fc ? cols : rows;
    for (int64_t y = 0; y < c; ++y)
      for (int64_t x = 0; x < a; ++x)
        if (!fn(o.off + x + y * (int64_t)o.ld)) return false;
    return true;
  };
  for (const Group &G : p.groups) {
    int cur_rect = -1;
    int64_t rect_lo = 0, rect_hi = 0;
    for (int li : G.launches) {
      const Launch &L = p.launches[li];
      if (L.rect != cur_rect) {   // a new rectangle reuses the group's arena from scratch
        cur_rect = L.rect;
        rect_lo = (int64_t)(G.arena_off / (size_t)p.es);
        rect_hi = (int64_t)((G.arena_off + G.arena_bytes) / (size_t)p.es);
        std::fill(ws.begin() + rect_lo, ws.begin() + rect_hi, 0);
        // the per-k loop: every rectangle is one more pass over C; the first
        // writes each element once, a later one each at most once
        if (per_k && L.rect > 0) std::fill(cbits.begin(), cbits.end(), 0);
      }
      // workspace marks: the writer's stage.  A stage reads what earlier
      // stages of its rectangle wrote; the side launch runs beside stages 1
      // and 2, so only the final update may read it, and it reads no workspace
      const uint8_t me = (uint8_t)L.stage;
      auto readable = [&](uint8_t w) {
        if (w == 0 || me == STAGE_SIDE) return false;
        return w == STAGE_SIDE ? me == 3 : w < me;
      };
      // collect distinct tasks of the launch
      std::vector<int32_t> tl;
      for (int64_t e = L.tile_off; e < L.tile_off + L.n_tiles; ++e)
        if (p.tiles[e].task >= 0) tl.push_back(p.tiles[e].task);
      std::sort(tl.begin(), tl.end());
      tl.erase(std::unique(tl.begin(), tl.end()), tl.end());
      for (int32_t ti : tl) {
        const DevTask &d = p.tasks[ti];
        for (int s = 0; s < d.nseg; ++s) {
          for (int w = 0; w < 2; ++w) {
            const DevOperand &o = w == 0 ? d.seg[s].a : d.seg[s].b;
            if (o.base != BASE_WS) continue;
            bool ok = w == 0 ? for_elems(o, d.M, d.seg[s].K, [&](int64_t e) {
                                 return e >= rect_lo && e < rect_hi && readable(ws[e]);
                               })
                             : for_elems(o, d.seg[s].K, d.N, [&](int64_t e) {
                                 return e >= rect_lo && e < rect_hi && readable(ws[e]);
                               });
            if (!ok) return fail(TLR_ERR_INVALID_ARG, "internal: workspace read before it is written (task " + std::to_string(ti) + ")");
          }
        }
        for (int n = 0; n < d.N; ++n) {
          int64_t col = d.ctab < 0 ? (int64_t)n * d.ldc : p.coltab[d.ctab + n];
          for (int m = 0; m < d.M; ++m) {
            int64_t e = d.c_off + col + m;
            if (d.c_base == BASE_WS) {
              if (e < rect_lo || e >= rect_hi || ws[e] != 0)
                return fail(TLR_ERR_INVALID_ARG, "internal: overlapping workspace writes (task " + std::to_string(ti) + ")");
              ws[e] = me;
            } else if (d.c_base == BASE_C) {
              uint64_t &word = cbits[(size_t)e >> 6];
              uint64_t bit = 1ull << (e & 63);
              if (word & bit) return fail(TLR_ERR_INVALID_ARG, "internal: element of C written twice");
              if (e % p.ldc >= p.m) return fail(TLR_ERR_INVALID_ARG, "internal: write into C's padding");
              word |= bit;
              if (!per_k || L.rect == 0) cwrites++;
            } else {
              return fail(TLR_ERR_INVALID_ARG, "internal: task writes an input buffer");
            }
          }
        }
      }
    }
  }
  if (cwrites != p.m * p.n) return fail(TLR_ERR_INVALID_ARG, "internal: C not covered exactly once");
  return TLR_OK;
}

// The per-contraction-tile loop ("Many small GEMMs"): for each k, launch 1
// forms the couplings S_ij = V_ik^T W_kj (and, at dense diagonal tiles,
// X_j = op(D_A,kk) W_kj and Y_i = V_ik^T op(D_B,kk)), launch 2 the right
// products T_ij = S_ij Z_kj^T, and launch 3 adds U_ik T_ij (or X_j Z_kj^T,
// U_ik Y_i, op(D_A,kk) op(D_B,kk)) into every output tile, with the caller's
// beta in the first pass and beta = 1 after: one pass over C per k.  Each k
// is one rectangle over all of C reusing the workspace of the previous one.
static tlr_status build_per_k(Plan &p, const Sums &s) {
  const View &A = p.A, &B = p.B;
  const int qm = s.qm, qk = s.qk, qn = s.qn;
  const int64_t es = p.es, b = A.b;
  p.rects.clear();
  p.groups.clear();
  if (qm == 0 || qn == 0) return TLR_OK;
  // workspace of one pass (every buffer 256-B aligned, slots at even offsets)
  struct Slots { std::vector<int64_t> S, T, X, Y; size_t bytes = 0; };
  auto slots = [&](int k, Slots &o) {
    o.S.assign((size_t)qm * qn, -1);
    o.T.assign((size_t)qm * qn, -1);
    o.X.assign(qn, -1);
    o.Y.assign(qm, -1);
    int64_t cur = 0;
    auto take = [&](int64_t elems) { int64_t off = cur; cur += even_up(elems); return off; };
    for (int i = 0; i < qm; ++i)
      for (int j = 0; j < qn; ++j) {
        const bool ad = A.diag && i == k, bd = B.diag && k == j;
        if (!ad && !bd && A.r(i, k) > 0 && B.r(k, j) > 0) {
          o.S[(size_t)i + (size_t)j * qm] = take((int64_t)A.r(i, k) * B.r(k, j));
          o.T[(size_t)i + (size_t)j * qm] = take((int64_t)A.r(i, k) * p.ns[j]);
        }
      }
    for (int j = 0; j < qn; ++j)
      if (A.diag && k < qm && !(B.diag && k == j) && B.r(k, j) > 0) o.X[j] = take(A.rs[k] * (int64_t)B.r(k, j));
    for (int i = 0; i < qm; ++i)
      if (B.diag && k < qn && !(A.diag && i == k) && A.r(i, k) > 0) o.Y[i] = take((int64_t)A.r(i, k) * p.ns[k]);
    o.bytes = align_up((size_t)cur * (size_t)es, WS_ALIGN);
  };
  size_t need = 0;
  for (int k = 0; k < qk; ++k) { Slots o; slots(k, o); need = std::max(need, o.bytes); }
  if (p.budget && need > p.budget)
    return fail(TLR_ERR_WORKSPACE, "the per-k loop needs " + std::to_string(need) + " B of workspace");
  Group G;
  G.stream = 0;
  G.arena_off = 0;
  G.arena_bytes = need;
  p.groups.push_back(G);
  p.ws_bytes = need;
  for (int k = 0; k < qk; ++k) {
    Slots o;
    slots(k, o);
    const int rect = (int)p.rects.size();
    p.rects.push_back(Rect{0, qm, 0, qn, TLR_ORDER_RIGHT, 0, o.bytes, 0});
    p.groups[0].rects.push_back(rect);
    TaskList l1, l2, l3;
    const int64_t sk = A.cs[k];
    for (int i = 0; i < qm; ++i)
      for (int j = 0; j < qn; ++j) {
        const size_t ij = (size_t)i + (size_t)j * qm;
        if (o.S[ij] < 0) continue;
        const int32_t ra = A.r(i, k), rb = B.r(k, j);
        DevTask d = new_task(ra, rb, BASE_WS, o.S[ij], ra, -1, false);
        add_seg(d, opnd(A.inner_base, A.ic(i, k) * b, b, 1), opnd(B.outer_base, B.oc(k, j) * b, b, 0), sk);
        l1.t.push_back(d);
        l1.useful.push_back(2.0 * ra * (double)rb * sk);
        DevTask e = new_task(ra, p.ns[j], BASE_WS, o.T[ij], ra, -1, false);
        add_seg(e, opnd(BASE_WS, o.S[ij], ra, 0), opnd(B.inner_base, B.ic(k, j) * b, b, 1), rb);
        l2.t.push_back(e);
        l2.useful.push_back(2.0 * ra * (double)p.ns[j] * rb);
      }
    for (int j = 0; j < qn; ++j)
      if (o.X[j] >= 0) {
        DevTask d = new_task(A.rs[k], B.r(k, j), BASE_WS, o.X[j], A.rs[k], -1, false);
        add_seg(d, opnd(A.diag_base, (int64_t)k * b * b, b, A.diag_trans), opnd(B.outer_base, B.oc(k, j) * b, b, 0), sk);
        l1.t.push_back(d);
        l1.useful.push_back(2.0 * A.rs[k] * (double)B.r(k, j) * sk);
      }
    for (int i = 0; i < qm; ++i)
      if (o.Y[i] >= 0) {
        DevTask d = new_task(A.r(i, k), p.ns[k], BASE_WS, o.Y[i], A.r(i, k), -1, false);
        add_seg(d, opnd(A.inner_base, A.ic(i, k) * b, b, 1), opnd(B.diag_base, (int64_t)k * b * b, b, B.diag_trans), sk);
        l1.t.push_back(d);
        l1.useful.push_back(2.0 * A.r(i, k) * (double)p.ns[k] * sk);
      }
    for (int j = 0; j < qn; ++j)
      for (int i = 0; i < qm; ++i) {
        DevTask d = new_task(A.rs[i], p.ns[j], BASE_C, A.ro[i] + p.no[j] * p.ldc, p.ldc, -1, true);
        const size_t ij = (size_t)i + (size_t)j * qm;
        const bool ad = A.diag && i == k, bd = B.diag && k == j;
        double u = 0;
        if (ad && bd) {
          add_seg(d, opnd(A.diag_base, (int64_t)k * b * b, b, A.diag_trans), opnd(B.diag_base, (int64_t)k * b * b, b, B.diag_trans), sk);
          u = 2.0 * A.rs[i] * (double)p.ns[j] * sk;
        } else if (ad) {
          if (o.X[j] >= 0) {
            add_seg(d, opnd(BASE_WS, o.X[j], A.rs[k], 0), opnd(B.inner_base, B.ic(k, j) * b, b, 1), B.r(k, j));
            u = 2.0 * A.rs[i] * (double)p.ns[j] * B.r(k, j);
          }
        } else if (bd) {
          if (o.Y[i] >= 0) {
            add_seg(d, opnd(A.outer_base, A.oc(i, k) * b, b, 0), opnd(BASE_WS, o.Y[i], A.r(i, k), 0), A.r(i, k));
            u = 2.0 * A.rs[i] * (double)p.ns[j] * A.r(i, k);
          }
        } else if (o.S[ij] >= 0) {
          add_seg(d, opnd(A.outer_base, A.oc(i, k) * b, b, 0), opnd(BASE_WS, o.T[ij], A.r(i, k), 0), A.r(i, k));
          u = 2.0 * A.rs[i] * (double)p.ns[j] * A.r(i, k);
        }
        // a later pass skips tiles without a term; the first pass writes every
        // tile (beta C alone where there is none)
        if (d.nseg == 0 && k > 0) continue;
        l3.t.push_back(d);
        l3.useful.push_back(u);
      }
    double F = 0;
    for (double x : l1.useful) F += x;
    for (double x : l2.useful) F += x;
    for (double x : l3.useful) F += x;
    p.rects[rect].useful_flops = F;
    emit_launch(p, 1, 0, rect, l1);
    emit_launch(p, 2, 0, rect, l2);
    const int c = emit_launch(p, 3, 0, rect, l3);
    if (c >= 0 && k > 0) p.launches[c].beta_one = true;
  }
  return TLR_OK;
}

// 16-bit types: the kernel moves operands in 16-byte vectors of 8 elements
// along each operand's contiguous index, so every extent, offset and leading
// dimension it meets must be a multiple of 8.  The stored ranks (rounded up to
// a multiple of 8 by the caller, "Packing for the contraction"), the tile
// size, the matrix dimensions and the leading dimensions being multiples of 8
// makes every rank sum, tile size and workspace offset one.
static tlr_status check_16bit(const Plan &p) {
  auto m8 = [](int64_t x) { return x % 8 == 0; };
  const char *why = nullptr;
  // (a leading dimension matters only when its matrix has elements)
  if (!m8(p.m) || !m8(p.n) || !m8(p.k)) why = "16-bit types: every matrix dimension must be a multiple of 8";
  else if (p.m > 0 && p.n > 0 && !m8(p.ldc)) why = "16-bit types: ldc must be a multiple of 8";
  else if ((p.dense_a || p.dense_b) &&
           (!m8(p.dense_rows) || !m8(p.dense_cols) || (p.dense_rows > 0 && p.dense_cols > 0 && !m8(p.ldb))))
    why = "16-bit types: the dense operand's dimensions and leading dimension must be multiples of 8";
  if (why) return fail(TLR_ERR_INVALID_ARG, why);
  for (const View *v : {&p.A, &p.B}) {
    if ((v == &p.A && p.dense_a) || (v == &p.B && p.dense_b)) continue;
    if (!m8(v->b)) return fail(TLR_ERR_INVALID_ARG, "16-bit types: the tile size must be a multiple of 8");
    for (int32_t r : v->R)
      if (!m8(r)) return fail(TLR_ERR_RANK, "16-bit types: every stored rank must be a multiple of 8");
  }
  return TLR_OK;
}

// The same condition on the built descriptors (a safety net: it follows from
// check_16bit, and the kernel relies on it for in-bounds vector accesses).
static tlr_status check_16bit_tasks(const Plan &p) {
  auto m8 = [](int64_t x) { return x % 8 == 0; };
  for (const DevTask &t : p.tasks) {
    bool ok = m8(t.M) && m8(t.N) && m8(t.c_off) && (t.ctab >= 0 || m8(t.ldc));
    if (t.ctab >= 0)
      for (int n = 0; n < t.N && ok; ++n) ok = m8(p.coltab[t.ctab + n]);
    for (int g = 0; g < t.nseg && ok; ++g) {
      const DevSeg &d = t.seg[g];
      ok = m8(d.K) && m8(d.a.off) && m8(d.a.ld) && m8(d.b.off) && m8(d.b.ld);
    }
    if (!ok) return fail(TLR_ERR_INVALID_ARG, "internal: a 16-bit task is not 8-element aligned");
  }
  return TLR_OK;
}

tlr_status build_plan(tlr_dtype dt, tlr_op opA, const tlr_shape *A, tlr_op opB, const tlr_shape *B,
                      int64_t dense_rows, int64_t dense_cols, int64_t ldb, int64_t ldc, size_t budget,
                      int n_streams, uint32_t flags, bool build_descriptors, Plan *p) {
  if (dt != TLR_F32 && dt != TLR_F64 && dt != TLR_F16 && dt != TLR_BF16)
    return fail(TLR_ERR_INVALID_ARG, "dtype must be TLR_F32, TLR_F64, TLR_F16 or TLR_BF16");
  if ((opA != TLR_OP_N && opA != TLR_OP_T) || (opB != TLR_OP_N && opB != TLR_OP_T))
    return fail(TLR_ERR_INVALID_ARG, "op must be TLR_OP_N or TLR_OP_T");
  if (n_streams < 1) return fail(TLR_ERR_INVALID_ARG, "n_streams must be >= 1");
  if ((flags & TLR_PLAN_FORCE_RIGHT) && (flags & TLR_PLAN_FORCE_LEFT))
    return fail(TLR_ERR_INVALID_ARG, "cannot force both orders");
  if (flags & ~(TLR_PLAN_FORCE_RIGHT | TLR_PLAN_FORCE_LEFT | TLR_PLAN_NO_REGIONS | TLR_PLAN_VALIDATE | TLR_PLAN_PIPELINE |
                TLR_PLAN_PER_K))
    return fail(TLR_ERR_INVALID_ARG, "unknown flag bits");
  if ((flags & TLR_PLAN_PIPELINE) && n_streams < 2)
    return fail(TLR_ERR_INVALID_ARG, "pipelining needs n_streams >= 2");
  p->dt = dt;
  p->es = dt == TLR_F64 ? 8 : (dt == TLR_F32 ? 4 : 2);
  p->budget = budget;
  p->n_streams = n_streams;
  p->flags = flags;
  p->dense_b = (B == nullptr);
  p->dense_a = (A == nullptr);
  p->opA = opA;
  p->opB = opB;
  if (p->dense_a && p->dense_b) return fail(TLR_ERR_INVALID_ARG, "A and B cannot both be dense (one TLR operand needed)");
  tlr_status st = TLR_OK;
  if (p->dense_a) {
    // dense A (stored dense_rows x dense_cols, leading dim ldb) times a TLR B
    if (flags & TLR_PLAN_FORCE_RIGHT) return fail(TLR_ERR_UNSUPPORTED, "the right order needs a TLR A");
    if (flags & TLR_PLAN_PIPELINE) return fail(TLR_ERR_UNSUPPORTED, "pipelining needs a TLR A");
    if (dense_rows < 0 || dense_cols < 0) return fail(TLR_ERR_INVALID_ARG, "bad dense A dims");
    st = make_view(B, opB, BASE_B_OUTER, BASE_B_INNER, BASE_B_DIAG, "B", &p->B);
    if (st != TLR_OK) return st;
    p->m = opA == TLR_OP_N ? dense_rows : dense_cols;
    p->k = opA == TLR_OP_N ? dense_cols : dense_rows;
    const int64_t kb = opB == TLR_OP_N ? B->rows : B->cols;
    p->n = opB == TLR_OP_N ? B->cols : B->rows;
    if (kb != p->k) return fail(TLR_ERR_INVALID_ARG, "op(A) columns != op(B) rows");
    if (ldb < std::max<int64_t>(1, dense_rows)) return fail(TLR_ERR_INVALID_ARG, "lda < rows of A");
    if (ldb >= (int64_t)1 << 21) return fail(TLR_ERR_INVALID_ARG, "lda must be below 2^21");
    p->ldb = ldb;
    p->dense_rows = dense_rows;
    p->dense_cols = dense_cols;
    // A as a view without ranks: row tiles of op(A) of B's tile size,
    // contraction tiles those of op(B)'s rows
    View &V = p->A;
    V.b = B->b;
    split_dim(p->m, B->b, V.rs, V.ro);
    V.cs = p->B.rs;
    V.co = p->B.ro;
    V.qr = (int)V.rs.size();
    V.qc = (int)V.cs.size();
    V.R.assign((size_t)V.qr * V.qc, 0);
    V.ocol.assign((size_t)V.qr * V.qc, 0);
    V.icol.assign((size_t)V.qr * V.qc, 0);
    V.diag = false;
    V.outer_base = BASE_A_OUTER;
    V.inner_base = BASE_A_INNER;
    V.diag_base = BASE_A_DIAG;
    p->ns = p->B.cs;
    p->no = p->B.co;
  } else {
    st = make_view(A, opA, BASE_A_OUTER, BASE_A_INNER, BASE_A_DIAG, "A", &p->A);
    if (st != TLR_OK) return st;
    p->m = opA == TLR_OP_N ? A->rows : A->cols;
    p->k = opA == TLR_OP_N ? A->cols : A->rows;
  }
  if (p->dense_a) {
  } else if (p->dense_b) {
    if (flags & TLR_PLAN_FORCE_LEFT) return fail(TLR_ERR_UNSUPPORTED, "the left order needs a TLR B");
    if (dense_rows < 0 || dense_cols < 0) return fail(TLR_ERR_INVALID_ARG, "bad dense B dims");
    int64_t kb = opB == TLR_OP_N ? dense_rows : dense_cols;
    p->n = opB == TLR_OP_N ? dense_cols : dense_rows;
    if (kb != p->k) return fail(TLR_ERR_INVALID_ARG, "op(A) columns != op(B) rows");
    if (ldb < std::max<int64_t>(1, dense_rows)) return fail(TLR_ERR_INVALID_ARG, "ldb < rows of B");
    if (ldb >= (int64_t)1 << 21) return fail(TLR_ERR_INVALID_ARG, "ldb must be below 2^21");
    p->ldb = ldb;
    p->dense_rows = dense_rows;
    p->dense_cols = dense_cols;
    split_dim(p->n, p->A.b, p->ns, p->no);
  } else {
    st = make_view(B, opB, BASE_B_OUTER, BASE_B_INNER, BASE_B_DIAG, "B", &p->B);
    if (st != TLR_OK) return st;
    if (B->b != A->b) return fail(TLR_ERR_INVALID_ARG, "A and B must use the same tile size");
    int64_t kb = opB == TLR_OP_N ? B->rows : B->cols;
    p->n = opB == TLR_OP_N ? B->cols : B->rows;
    if (kb != p->k) return fail(TLR_ERR_INVALID_ARG, "op(A) columns != op(B) rows");
    p->ns = p->B.cs;
    p->no = p->B.co;
  }
  if (ldc < std::max<int64_t>(1, p->m)) return fail(TLR_ERR_INVALID_ARG, "ldc < rows of C");
  if (ldc > std::numeric_limits<int32_t>::max()) return fail(TLR_ERR_INVALID_ARG, "ldc too large");
  if (p->m > std::numeric_limits<int32_t>::max() || p->n > std::numeric_limits<int32_t>::max())
    return fail(TLR_ERR_INVALID_ARG, "C dimensions too large");
  p->ldc = ldc;
  if (p->es == 2) {
    st = check_16bit(*p);
    if (st != TLR_OK) return st;
  }

  Sums s;
  build_sums(*p, s);
  const int qm = s.qm, qn = s.qn;
  // whole-C accounting
  p->flops_right = p->dense_a ? -1 : ((qm && qn) ? rect_useful(*p, s, 0, qm, 0, qn, TLR_ORDER_RIGHT) : 0);
  p->flops_left = p->dense_b ? -1 : ((qm && qn) ? rect_useful(*p, s, 0, qm, 0, qn, TLR_ORDER_LEFT) : 0);
  p->final_right = p->dense_a ? -1 : 0;
  if (!p->dense_a)
    for (int i = 0; i < qm; ++i) p->final_right += 2.0 * p->A.rs[i] * (double)s.rho[i] * p->n;
  if (!p->dense_b) {
    p->final_left = 0;
    for (int j = 0; j < qn; ++j) p->final_left += 2.0 * p->ns[j] * (double)s.gam[j] * p->m;
  }
  p->alg_bytes = (double)p->es * ((p->dense_a ? (double)dense_rows * dense_cols : compressed_elems(p->A)) +
                                  (p->dense_b ? (double)dense_rows * dense_cols : compressed_elems(p->B)) +
                                  (double)p->m * p->n);

  const bool per_k = (flags & TLR_PLAN_PER_K) != 0;
  if (per_k) {
    if (p->dense_a || p->dense_b) return fail(TLR_ERR_UNSUPPORTED, "the per-k loop needs two TLR operands");
    if (flags & (TLR_PLAN_PIPELINE | TLR_PLAN_FORCE_LEFT))
      return fail(TLR_ERR_UNSUPPORTED, "the per-k loop takes neither pipelining nor the left order");
    p->tasks.clear();
    p->tiles.clear();
    p->coltab.clear();
    p->launches.clear();
    st = build_per_k(*p, s);
    if (st != TLR_OK) return st;
  } else {
    st = schedule(*p, s);
    if (st != TLR_OK) return st;
  }
  p->useful_flops = 0;
  for (auto &r : p->rects) p->useful_flops += r.useful_flops;
  if (!build_descriptors) return TLR_OK;

  if (!per_k) {
    p->tasks.clear();
    p->tiles.clear();
    p->coltab.clear();
    p->launches.clear();
    for (size_t g = 0; g < p->groups.size(); ++g)
      for (int r : p->groups[g].rects) emit_rect(*p, s, r);
  }
  // output columns that start on a 16-byte boundary allow 16-byte C accesses
  const int64_t vec_el = 16 / p->es;
  for (DevTask &d : p->tasks) {
    bool v = d.c_off % vec_el == 0;
    if (d.ctab < 0) v = v && d.ldc % vec_el == 0;
    else
      for (int n = 0; n < d.N && v; ++n) v = p->coltab[d.ctab + n] % vec_el == 0;
    d.flags = v ? TASK_VEC : 0;
  }
  // pipelining: the second stream starts once the first rectangle's stage 2
  // (its last launch before the final update) is done, so that its first
  // stages run beside that final update
  if ((flags & TLR_PLAN_PIPELINE) && p->groups.size() == 2 && !p->groups[1].launches.empty()) {
    int dep = -1;
    for (int l : p->groups[0].launches)
      if (p->launches[l].rect == p->groups[0].rects[0] && p->launches[l].stage < 3) dep = l;
    p->launches[p->groups[1].launches[0]].wait_launch = dep;
  }
  if (p->es == 2) {
    st = check_16bit_tasks(*p);
    if (st != TLR_OK) return st;
  }
  p->executed_flops = 0;
  for (auto &L : p->launches) p->executed_flops += L.executed_flops;
  p->task_bytes_off = 0;
  p->tile_bytes_off = align_up(p->tasks.size() * sizeof(DevTask), WS_ALIGN);
  p->ctab_bytes_off = p->tile_bytes_off + align_up(p->tiles.size() * sizeof(DevTile), WS_ALIGN);
  p->desc_bytes = p->ctab_bytes_off + align_up(p->coltab.size() * sizeof(int64_t), WS_ALIGN);
  if (p->desc_bytes == 0) p->desc_bytes = WS_ALIGN;
  return validate(*p, (flags & TLR_PLAN_VALIDATE) != 0);
}

}  // namespace tlr
