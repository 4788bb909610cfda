// Device descriptors of the grouped GEMM launches (shared by planner and kernel).
//
// Every launch runs a list of GEMM tasks; every task computes one output
// block C (M x N, column-major) as the sum of up to two K segments
//   acc = sum_seg  opnd(A_seg) (M x K_seg) * opnd(B_seg) (K_seg x N)
// and stores  C = alpha*acc + beta*C  (final tasks, the dense update of C) or
// C = acc (intermediates in the workspace).  A launch is a flat table of
// workgroup entries (task, m0, n0), one per BM x BN block of some task.
//
// Operand addressing: element (r, c) of an A operand (M x K) is
//   trans == 0 : base[off + r + c*ld]      (column-major, M contiguous)
//   trans == 1 : base[off + c + r*ld]      (K contiguous)
// and of a B operand (K x N)
//   trans == 0 : base[off + r + c*ld]      (column-major, K contiguous)
//   trans == 1 : base[off + c + r*ld]      (N contiguous).
// Output element (m, n) lives at C_base[c_off + m + col(n)] with
// col(n) = n*ldc (ctab < 0) or col(n) = coltab[ctab + n] (an indirect column
// map: how the right product writes each coupling row straight into the
// terminal matrix of its tile row).
#pragma once
#include <stdint.h>

namespace tlr {

enum BaseId : uint8_t {
  BASE_A_OUTER = 0, BASE_A_INNER = 1, BASE_A_DIAG = 2,
  BASE_B_OUTER = 3, BASE_B_INNER = 4, BASE_B_DIAG = 5,
  BASE_B_DENSE = 6, BASE_WS = 7, BASE_C = 8, NUM_BASES = 9
};

struct DevOperand {      // 16 bytes
  int64_t off;
  int32_t ld;
  uint8_t base;
  uint8_t trans;
  uint16_t flags;        // OperandFlags
};

// OPND_PADDED: ld exceeds the extent along the contiguous index and the buffer
// holds every ld-strided vector whole, so the element one past that extent is
// addressable (its value is unspecified).
enum OperandFlags : uint16_t { OPND_PADDED = 1 };

struct DevSeg {          // 40 bytes
  DevOperand a;
  DevOperand b;
  int32_t K;
  int32_t pad;
};

struct DevTask {         // 112 bytes
  int32_t M, N;
  int64_t c_off;
  int64_t ctab;          // < 0: affine columns
  int32_t ldc;
  uint8_t c_base;
  uint8_t final_;        // 1: alpha/beta update of C
  uint8_t nseg;
  uint8_t flags;         // TASK_VEC: every output column starts 16-byte aligned
  DevSeg seg[2];
};

enum TaskFlags : uint8_t { TASK_VEC = 1 };

// How the kernel loads the first K segment of a task (a launch's workgroup
// table is split into one contiguous sub-table per mode).  The pair modes load
// two adjacent elements per instruction: along M (PAIR_M, A M-contiguous) or
// along K (PAIR_K, A K-contiguous) for A, and along the contiguous index for B.
// A task qualifies for a pair mode when, for both operands of that segment,
// the element offset and the leading dimension are even (the buffer bases must
// be aligned to a pair, checked when the plan runs) and every pair either lies
// inside the operand or outside it, or straddles the end of an M or N extent
// into a padded operand: the extra element then only feeds a row or column of
// the output that is never stored.  Along K both elements of a pair must be
// real, since the extra one would multiply the other operand's zero.
enum LoadMode : int { LOAD_SINGLE = 0, LOAD_PAIR_M = 1, LOAD_PAIR_K = 2, NUM_LOAD_MODES = 3 };

inline int task_load_mode(const DevTask &t) {
  if (t.nseg < 1) return LOAD_SINGLE;
  const DevSeg &s = t.seg[0];
  const bool b_ok = (s.b.off % 2) == 0 && (s.b.ld % 2) == 0 &&
                    (s.b.trans == 1 ? (t.N % 2) == 0 || (s.b.flags & OPND_PADDED) : (s.K % 2) == 0);
  const bool a_ok = (s.a.off % 2) == 0 && (s.a.ld % 2) == 0;
  if (!a_ok || !b_ok) return LOAD_SINGLE;
  if (s.a.trans == 0) return (t.M % 2) == 0 || (s.a.flags & OPND_PADDED) ? LOAD_PAIR_M : LOAD_SINGLE;
  return (s.K % 2) == 0 ? LOAD_PAIR_K : LOAD_SINGLE;
}

struct DevTile {         // 16 bytes
  int32_t task;          // < 0: idle workgroup (launch padding)
  int32_t m0, n0;
  int32_t pad;
};

struct Bases {
  const void *p[NUM_BASES];
};

static_assert(sizeof(DevOperand) == 16, "DevOperand layout");
static_assert(sizeof(DevSeg) == 40, "DevSeg layout");
static_assert(sizeof(DevTask) == 112, "DevTask layout");
static_assert(sizeof(DevTile) == 16, "DevTile layout");

}  // namespace tlr
