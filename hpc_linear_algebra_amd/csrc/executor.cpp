// Device side of a plan: descriptor upload, the launch sequence of one product,
// stream fork/join for concurrent regions, per-launch event timing, and the
// dense GEMM entry.
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "tlr_plan.h"

namespace tlr {

static bool bases_pair_aligned(const Bases &b, int es) {
  for (const void *x : b.p)
    if (reinterpret_cast<uintptr_t>(x) % (uintptr_t)(2 * es) != 0) return false;
  return true;
}


#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) return fail(TLR_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

static void destroy_events(std::vector<void *> &ev) {
  for (void *e : ev)
    if (e) (void)hipEventDestroy(static_cast<hipEvent_t>(e));
  ev.clear();
}

void plan_release_device(Plan *p) {
  destroy_events(p->join_events);
  destroy_events(p->dep_events);
  destroy_events(p->prof_events);
  destroy_events(p->mode_events);
  destroy_events(p->side_events);
  destroy_events(p->side_join);
  p->forks_at.clear();
  for (void *s : p->aux_streams)
    if (s) (void)hipStreamDestroy(static_cast<hipStream_t>(s));
  p->aux_streams.clear();
  if (p->fork_event) {
    (void)hipEventDestroy(static_cast<hipEvent_t>(p->fork_event));
    p->fork_event = nullptr;
  }
  p->dev_desc = nullptr;
}

Plan::~Plan() { plan_release_device(this); }

tlr_status plan_bind(Plan *p, void *dev, size_t bytes, void *stream) {
  if (!dev) return fail(TLR_ERR_INVALID_ARG, "bind: null descriptor buffer");
  if (bytes < p->desc_bytes) return fail(TLR_ERR_INVALID_ARG, "bind: descriptor buffer too small");
  if (reinterpret_cast<uintptr_t>(dev) % WS_ALIGN) return fail(TLR_ERR_INVALID_ARG, "bind: buffer not 256-byte aligned");
  std::vector<char> h(p->desc_bytes, 0);
  if (!p->tasks.empty()) std::memcpy(h.data() + p->task_bytes_off, p->tasks.data(), p->tasks.size() * sizeof(DevTask));
  if (!p->tiles.empty()) std::memcpy(h.data() + p->tile_bytes_off, p->tiles.data(), p->tiles.size() * sizeof(DevTile));
  if (!p->coltab.empty()) std::memcpy(h.data() + p->ctab_bytes_off, p->coltab.data(), p->coltab.size() * sizeof(int64_t));
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(hipMemcpyAsync(dev, h.data(), p->desc_bytes, hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  plan_release_device(p);
  int devno = 0;
  HIP_TRY(hipGetDevice(&devno));
  hipEvent_t fe;
  HIP_TRY(hipEventCreateWithFlags(&fe, hipEventDisableTiming));
  p->fork_event = fe;
  for (size_t g = 0; g < p->groups.size(); ++g) {
    hipEvent_t je;
    HIP_TRY(hipEventCreateWithFlags(&je, hipEventDisableTiming));
    p->join_events.push_back(je);
  }
  for (size_t l = 0; l < p->launches.size(); ++l) {
    hipEvent_t de = nullptr;
    bool awaited = false;
    for (const Launch &L : p->launches) awaited = awaited || L.wait_launch == (int)l;
    if (awaited) HIP_TRY(hipEventCreateWithFlags(&de, hipEventDisableTiming));
    p->dep_events.push_back(de);
  }
  bool split = false;
  for (size_t l = 0; l < p->launches.size(); ++l) {
    const Launch &L = p->launches[l];
    int parts = 0;
    for (int m = 0; m < NUM_LOAD_MODES; ++m) parts += L.mode_tiles[m] > 0;
    for (int e = 0; e < 3; ++e) {
      hipEvent_t me = nullptr;
      if (parts > 1) HIP_TRY(hipEventCreateWithFlags(&me, hipEventDisableTiming));
      p->mode_events.push_back(me);
    }
    split = split || parts > 1;
  }
  bool side = false;
  p->forks_at.assign(p->launches.size(), {});
  for (size_t l = 0; l < p->launches.size(); ++l) {
    const Launch &L = p->launches[l];
    hipEvent_t se = nullptr;
    if (L.stage == STAGE_SIDE) {
      HIP_TRY(hipEventCreateWithFlags(&se, hipEventDisableTiming));
      p->forks_at[L.fork_at >= 0 ? (size_t)L.fork_at : l].push_back((int)l);
      side = true;
    }
    p->side_events.push_back(se);
  }
  for (size_t g = 0; g < p->groups.size(); ++g) {
    hipEvent_t je = nullptr;
    bool any = false;
    for (int l : p->groups[g].launches) any = any || p->launches[l].stage == STAGE_SIDE || p->launches[l].on_side;
    if (any) HIP_TRY(hipEventCreateWithFlags(&je, hipEventDisableTiming));
    p->side_join.push_back(je);
  }
  if (split || side)
    for (size_t i = 0; i < AUX_PER_GROUP * p->groups.size(); ++i) {
      hipStream_t as;
      HIP_TRY(hipStreamCreateWithFlags(&as, hipStreamNonBlocking));   // ordered by events only
      p->aux_streams.push_back(as);
    }
  p->device = devno;
  p->dev_desc = dev;
  return TLR_OK;
}

tlr_status plan_profile(Plan *p, int max_exec) {
  destroy_events(p->prof_events);
  p->prof_max = 0;
  p->prof_count = 0;
  if (max_exec <= 0) return TLR_OK;
  const size_t per = 2 * (p->launches.size() + 1);
  for (size_t e = 0; e < per * (size_t)max_exec; ++e) {
    hipEvent_t ev;
    HIP_TRY(hipEventCreate(&ev));
    p->prof_events.push_back(ev);
  }
  p->prof_max = max_exec;
  return TLR_OK;
}

tlr_status plan_profile_read(Plan *p, double *stage_ms, double *launch_ms, int32_t *execs) {
  for (int s = 0; s < 5; ++s) stage_ms[s] = 0;
  if (launch_ms)
    for (size_t l = 0; l < p->launches.size(); ++l) launch_ms[l] = 0;
  const size_t nl = p->launches.size();
  const size_t per = 2 * (nl + 1);
  for (int x = 0; x < p->prof_count; ++x) {
    for (size_t l = 0; l <= nl; ++l) {
      hipEvent_t a = static_cast<hipEvent_t>(p->prof_events[x * per + 2 * l]);
      hipEvent_t b = static_cast<hipEvent_t>(p->prof_events[x * per + 2 * l + 1]);
      float ms = 0;
      HIP_TRY(hipEventElapsedTime(&ms, a, b));
      if (l == nl) {
        stage_ms[3] += ms;
      } else {
        const int st = p->launches[l].stage;
        stage_ms[st == STAGE_SIDE ? 4 : st - 1] += ms;
        if (launch_ms) launch_ms[l] += ms;
      }
    }
  }
  *execs = p->prof_count;
  p->prof_count = 0;
  return TLR_OK;
}

static bool any_rank(const View &v) {
  for (int32_t r : v.R)
    if (r > 0) return true;
  return false;
}

tlr_status plan_execute(Plan *p, double alpha, const tlr_buffers *A, const tlr_buffers *B, const void *B_dense,
                        int64_t ldb, double beta, void *C, int64_t ldc, void *ws, size_t ws_bytes,
                        void *const *streams, int n_streams) {
  if (!p->dev_desc) return fail(TLR_ERR_NOT_BOUND, "execute: plan is not bound");
  if (n_streams < 1) return fail(TLR_ERR_INVALID_ARG, "execute: n_streams must be >= 1");
  if (ldc != p->ldc) return fail(TLR_ERR_INVALID_ARG, "execute: ldc differs from the analysed one");
  if (p->m > 0 && p->n > 0 && !C) return fail(TLR_ERR_INVALID_ARG, "execute: null C");
  if (!p->dense_a) {
    if (!A) return fail(TLR_ERR_INVALID_ARG, "execute: null A buffers");
    if (p->A.diag && p->A.qr > 0 && !A->diag) return fail(TLR_ERR_INVALID_ARG, "execute: null A diagonal");
    if (any_rank(p->A) && (!A->outer || !A->inner)) return fail(TLR_ERR_INVALID_ARG, "execute: null A factors");
  }
  if (p->dense_a || p->dense_b) {   // the dense operand
    if (ldb != p->ldb) return fail(TLR_ERR_INVALID_ARG, "execute: leading dimension of the dense operand differs from the analysed one");
    if (p->m > 0 && p->n > 0 && p->k > 0 && !B_dense) return fail(TLR_ERR_INVALID_ARG, "execute: null dense operand");
  }
  if (!p->dense_b) {
    if (!B) return fail(TLR_ERR_INVALID_ARG, "execute: null B buffers");
    if (p->B.diag && p->B.qr > 0 && !B->diag) return fail(TLR_ERR_INVALID_ARG, "execute: null B diagonal");
    if (any_rank(p->B) && (!B->outer || !B->inner)) return fail(TLR_ERR_INVALID_ARG, "execute: null B factors");
  }
  if (ws_bytes < p->ws_bytes) return fail(TLR_ERR_WORKSPACE, "execute: workspace smaller than the plan needs");
  if (p->ws_bytes > 0 && !ws) return fail(TLR_ERR_INVALID_ARG, "execute: null workspace");
  if (ws && reinterpret_cast<uintptr_t>(ws) % WS_ALIGN) return fail(TLR_ERR_INVALID_ARG, "execute: workspace not 256-byte aligned");
  int devno = 0;
  HIP_TRY(hipGetDevice(&devno));
  if (devno != p->device) return fail(TLR_ERR_INVALID_ARG, "execute: current device differs from the bound one");

  hipStream_t s0 = streams ? static_cast<hipStream_t>(streams[0]) : nullptr;
  if (p->m == 0 || p->n == 0) return TLR_OK;
  if (alpha == 0.0) {
    if (beta == 1.0) return TLR_OK;
    int e = launch_scale(p->dt, C, p->m, p->n, p->ldc, beta, s0);
    if (e) return fail(TLR_ERR_HIP, std::string("scale launch: ") + hipGetErrorString((hipError_t)e));
    return TLR_OK;
  }
  Bases bases;
  bases.p[BASE_A_OUTER] = A ? A->outer : nullptr;
  bases.p[BASE_A_INNER] = A ? A->inner : nullptr;
  bases.p[BASE_A_DIAG] = A ? A->diag : nullptr;
  bases.p[BASE_B_OUTER] = B ? B->outer : nullptr;
  bases.p[BASE_B_INNER] = B ? B->inner : nullptr;
  bases.p[BASE_B_DIAG] = B ? B->diag : nullptr;
  bases.p[BASE_B_DENSE] = B_dense;
  bases.p[BASE_WS] = ws;
  bases.p[BASE_C] = C;
  // the 16-bit kernel moves whole 16-byte vectors; the pair load modes of the
  // 32/64-bit kernel assume every buffer aligned to a pair of elements,
  // otherwise each launch runs its whole table in single-element mode (the
  // 16-bit kernel takes one launch per table, whatever the mode split)
  if (p->es == 2)
    for (const void *x : bases.p)
      if (reinterpret_cast<uintptr_t>(x) % 16 != 0)
        return fail(TLR_ERR_INVALID_ARG, "execute: 16-bit buffers must be 16-byte aligned");
  const bool pairs_ok = p->es != 2 && bases_pair_aligned(bases, p->es);
  const char *dd = static_cast<const char *>(p->dev_desc);
  const DevTask *tasks = reinterpret_cast<const DevTask *>(dd + p->task_bytes_off);
  const DevTile *tiles = reinterpret_cast<const DevTile *>(dd + p->tile_bytes_off);
  const int64_t *ctab = reinterpret_cast<const int64_t *>(dd + p->ctab_bytes_off);

  auto stream_of = [&](int g) -> hipStream_t {
    int si = p->groups[g].stream % n_streams;
    return streams ? static_cast<hipStream_t>(streams[si]) : nullptr;
  };
  auto aux = [&](int g, int i) { return static_cast<hipStream_t>(p->aux_streams[AUX_PER_GROUP * g + i]); };
  // the stream a launch runs on (its first load-mode part, for a split launch)
  auto launch_stream = [&](int l) -> hipStream_t {
    const Launch &L = p->launches[l];
    return L.stage == STAGE_SIDE || L.on_side ? aux(L.group, AUX_PER_GROUP - 1) : stream_of(L.group);
  };
  const bool prof = p->prof_count < p->prof_max;
  const size_t nl = p->launches.size();
  const size_t per = 2 * (nl + 1);
  auto pev = [&](size_t l, int which) {
    return static_cast<hipEvent_t>(p->prof_events[p->prof_count * per + 2 * l + which]);
  };
  if (prof) HIP_TRY(hipEventRecord(pev(nl, 0), s0));
  bool forked = false;
  for (size_t g = 0; g < p->groups.size(); ++g) {
    hipStream_t sg = stream_of((int)g);
    if (sg != s0) {
      if (!forked) {
        HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(p->fork_event), s0));
        forked = true;
      }
      HIP_TRY(hipStreamWaitEvent(sg, static_cast<hipEvent_t>(p->fork_event), 0));
    }
  }
  for (size_t g = 0; g < p->groups.size(); ++g) {
    hipStream_t sg = stream_of((int)g);
    for (int l : p->groups[g].launches) {
      const Launch &L = p->launches[l];
      const hipStream_t sl = launch_stream(l);
      if (L.wait_launch >= 0) {
        hipStream_t sw = launch_stream(L.wait_launch);
        if (sw != sl) HIP_TRY(hipStreamWaitEvent(sl, static_cast<hipEvent_t>(p->dep_events[L.wait_launch]), 0));
      }
      // side launches fork here: after everything enqueued on the group's
      // stream so far (earlier rectangles of the arena included), before l
      for (int d : p->forks_at[l]) HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(p->side_events[d]), sg));
      if (L.stage == STAGE_SIDE) {
        HIP_TRY(hipStreamWaitEvent(sl, static_cast<hipEvent_t>(p->side_events[l]), 0));
        if (prof) HIP_TRY(hipEventRecord(pev(l, 0), sl));
        // load-mode parts one after another on the side stream
        for (int m = 0; m < NUM_LOAD_MODES; ++m) {
          if (pairs_ok ? L.mode_tiles[m] == 0 : m > 0) continue;
          const int mode = pairs_ok ? m : LOAD_SINGLE;
          const int64_t off = pairs_ok ? L.mode_off[m] : 0, n = pairs_ok ? L.mode_tiles[m] : L.n_tiles;
          int e = launch_grouped(p->dt, L.stage, mode, L.bn, tasks, tiles + L.tile_off + off, n, ctab, bases, alpha,
                                 L.beta_one ? 1.0 : beta, sl);
          if (e) return fail(TLR_ERR_HIP, std::string("grouped GEMM launch: ") + hipGetErrorString((hipError_t)e));
        }
        if (prof) HIP_TRY(hipEventRecord(pev(l, 1), sl));
        if (p->dep_events[l]) HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(p->dep_events[l]), sl));
        continue;
      }
      if (prof) HIP_TRY(hipEventRecord(pev(l, 0), sl));
      if (pairs_ok) {
        // one kernel per load mode; several non-empty ones run side by side
        // (the first on the launch's stream, the others on the group's
        // auxiliary streams) so that a small sub-table does not run alone on
        // the GPU
        int part = 0;
        hipEvent_t fork = static_cast<hipEvent_t>(p->mode_events[3 * l]);
        if (fork) HIP_TRY(hipEventRecord(fork, sl));   // before the first sub-launch: all start together
        for (int m = 0; m < NUM_LOAD_MODES; ++m) {
          if (L.mode_tiles[m] == 0) continue;
          hipStream_t sm = sl;
          if (part > 0) {
            sm = aux(L.group, part - 1);
            HIP_TRY(hipStreamWaitEvent(sm, fork, 0));
          }
          int e = launch_grouped(p->dt, L.stage, m, L.bn, tasks, tiles + L.tile_off + L.mode_off[m], L.mode_tiles[m],
                                 ctab, bases, alpha, L.beta_one ? 1.0 : beta, sm);
          if (e) return fail(TLR_ERR_HIP, std::string("grouped GEMM launch: ") + hipGetErrorString((hipError_t)e));
          if (part > 0) {
            hipEvent_t join = static_cast<hipEvent_t>(p->mode_events[3 * l + part]);
            HIP_TRY(hipEventRecord(join, sm));
            HIP_TRY(hipStreamWaitEvent(sl, join, 0));
          }
          ++part;
        }
      } else {
        int e = launch_grouped(p->dt, L.stage, LOAD_SINGLE, L.bn, tasks, tiles + L.tile_off, L.n_tiles, ctab, bases,
                               alpha, L.beta_one ? 1.0 : beta, sl);
        if (e) return fail(TLR_ERR_HIP, std::string("grouped GEMM launch: ") + hipGetErrorString((hipError_t)e));
      }
      if (prof) HIP_TRY(hipEventRecord(pev(l, 1), sl));
      if (p->dep_events[l]) HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(p->dep_events[l]), sl));
    }
    if (p->side_join[g]) {   // every side launch of the group ends before the group does
      hipEvent_t je = static_cast<hipEvent_t>(p->side_join[g]);
      HIP_TRY(hipEventRecord(je, aux((int)g, AUX_PER_GROUP - 1)));
      HIP_TRY(hipStreamWaitEvent(sg, je, 0));
    }
  }
  for (size_t g = 0; g < p->groups.size(); ++g) {
    hipStream_t sg = stream_of((int)g);
    if (sg != s0) {
      hipEvent_t je = static_cast<hipEvent_t>(p->join_events[g]);
      HIP_TRY(hipEventRecord(je, sg));
      HIP_TRY(hipStreamWaitEvent(s0, je, 0));
    }
  }
  if (prof) {
    HIP_TRY(hipEventRecord(pev(nl, 1), s0));
    p->prof_count++;
  }
  return TLR_OK;
}

tlr_status dense_gemm(tlr_dtype dt, tlr_op opA, tlr_op opB, int64_t m, int64_t n, int64_t k, double alpha,
                      const void *A, int64_t lda, const void *B, int64_t ldb, double beta, void *C, int64_t ldc,
                      void *stream) {
  if (dt == TLR_F16 || dt == TLR_BF16) return fail(TLR_ERR_UNSUPPORTED, "dense: 16-bit types run only inside the TLR product");
  if (dt != TLR_F32 && dt != TLR_F64) return fail(TLR_ERR_INVALID_ARG, "dense: bad dtype");
  if ((opA != TLR_OP_N && opA != TLR_OP_T) || (opB != TLR_OP_N && opB != TLR_OP_T))
    return fail(TLR_ERR_INVALID_ARG, "dense: bad op");
  if (m < 0 || n < 0 || k < 0) return fail(TLR_ERR_INVALID_ARG, "dense: negative size");
  const int64_t lim = 0x7fffffff, ldlim = (int64_t)1 << 21;
  if (m > lim || n > lim || k > lim || lda >= ldlim || ldb >= ldlim || ldc > lim)
    return fail(TLR_ERR_INVALID_ARG, "dense: size or leading dim too large");
  const int64_t arows = opA == TLR_OP_N ? m : k, brows = opB == TLR_OP_N ? k : n;
  if (lda < std::max<int64_t>(1, arows) || ldb < std::max<int64_t>(1, brows) || ldc < std::max<int64_t>(1, m))
    return fail(TLR_ERR_INVALID_ARG, "dense: leading dimension too small");
  if (m == 0 || n == 0) return TLR_OK;
  if (!C) return fail(TLR_ERR_INVALID_ARG, "dense: null C");
  if (k > 0 && alpha != 0.0 && (!A || !B)) return fail(TLR_ERR_INVALID_ARG, "dense: null A or B");
  if (k == 0 || alpha == 0.0) {
    if (beta == 1.0) return TLR_OK;
    int e = launch_scale(dt, C, m, n, ldc, beta, stream);
    if (e) return fail(TLR_ERR_HIP, std::string("scale launch: ") + hipGetErrorString((hipError_t)e));
    return TLR_OK;
  }
  DevTask t;
  std::memset(&t, 0, sizeof(t));
  t.M = (int32_t)m;
  t.N = (int32_t)n;
  t.c_off = 0;
  t.ctab = -1;
  t.ldc = (int32_t)ldc;
  t.c_base = BASE_C;
  t.final_ = 1;
  t.nseg = 1;
  t.flags = ldc % (16 / (dt == TLR_F64 ? 8 : 4)) == 0 ? TASK_VEC : 0;
  t.seg[0].a.off = 0;
  t.seg[0].a.ld = (int32_t)lda;
  t.seg[0].a.base = BASE_A_OUTER;
  t.seg[0].a.trans = opA == TLR_OP_N ? 0 : 1;
  t.seg[0].b.off = 0;
  t.seg[0].b.ld = (int32_t)ldb;
  t.seg[0].b.base = BASE_B_OUTER;
  t.seg[0].b.trans = opB == TLR_OP_N ? 0 : 1;
  t.seg[0].K = (int32_t)k;
  Bases bases;
  for (auto &x : bases.p) x = nullptr;
  bases.p[BASE_A_OUTER] = A;
  bases.p[BASE_B_OUTER] = B;
  bases.p[BASE_C] = C;
  const int mode = bases_pair_aligned(bases, dt == TLR_F64 ? 8 : 4) ? task_load_mode(t) : LOAD_SINGLE;
  int e = launch_single(dt, mode, t, bases, alpha, beta, stream);
  if (e) return fail(TLR_ERR_HIP, std::string("dense GEMM launch: ") + hipGetErrorString((hipError_t)e));
  return TLR_OK;
}

}  // namespace tlr
