// Grouped, segmented-K MFMA GEMM for gfx950 (CDNA4), fp64 and fp32.
//
// One kernel body runs every stage of the TLR product: each workgroup reads one
// entry (task, m0, n0) of a launch's table and computes the 128 x 128 block of
// that task's output, accumulating over the task's K segments, then writes
// C = alpha*acc + beta*C (final update, C read only when beta != 0) or
// C = acc (workspace intermediates), through an affine or indirect column map.
// Layout of the descriptors: tlr_desc.h.  Each stage gets its own kernel symbol
// so that profilers report the stages separately.
//
// Work split: four wave64s stacked along M, each owning a 32 x 128 strip of
// the block as 2 x 8 MFMA tiles of 16 x 16 (v_mfma_f64_16x16x4_f64 /
// v_mfma_f32_16x16x4_f32).  K advances in stages of 16.  The A operand goes
// from global memory straight into registers in MFMA operand order (each wave
// loads its own 32 rows; no LDS round trip), refilled for the next stage as the
// current stage's MFMAs release each register.  The B operand, shared by all
// four waves, is staged through a three-buffer LDS ring, its global loads one
// stage ahead of the LDS store and the LDS fragments one k-step ahead of the
// MFMAs.  Registers are sized for two workgroups per CU (two waves per SIMD).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "tlr_plan.h"

namespace tlr {

namespace {

// LDS rows of the B tile hold 145 elements: an odd stride sends the 16 k-rows
// that one K-contiguous store touches to 16 different banks, and a 16-element
// fragment read still covers each bank once.
constexpr int KBM = 128, KBK = 16, KPAD = 17;
constexpr int NT = 256;               // threads per workgroup: four wave64s
constexpr int WM = 32;               // rows per wave: four waves stacked along M, 128 columns each
constexpr int MI = 2;                 // 16-row MFMA tiles per wave
// Block width: NJ 16-column MFMA tiles per wave (NJ = 8: 128 x 128 blocks,
// NJ = 4: 128 x 64 blocks with half the accumulators, for launches whose
// tasks are too few or too short to fill the chip with 128 x 128 blocks).
template <int NJ> struct Blk {
  static constexpr int KBN = 16 * NJ;             // block columns
  static constexpr int LDS_B = KBN + KPAD;        // LDS row stride of the B tile (odd)
  static constexpr int EPT = KBN * KBK / NT;      // B elements per thread per stage
  static constexpr int WAVES_PER_EU = NJ == 8 ? 2 : 3;
};

// Lane layout of the 16x16x4 MFMAs (measured on gfx950): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; accumulator element v of lane l is
// D[row][l % 16] with row = 4*(l/16) + v for fp32 but row = l/16 + 4*v for
// fp64.  Which row of the wave's slice of A enters MFMA row x is a free
// choice (A goes straight from memory to registers): arow(x) below is picked
// so that, after the MFMAs, the four lanes that share an output column hold
// one contiguous 16-byte unit each of a 64-byte run of that column.  One
// 16-byte store (or load) per lane then moves four whole 64-byte runs per
// column instead of sixteen-byte pieces scattered over four runs, which
// measured as 5.9 vs 3.4 TB/s for a pure store kernel of this block shape.
template <typename T> struct Mfma;
template <> struct Mfma<double> {
  typedef double v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 mma(double a, double b, v4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int arow(int x) { return x; }
};
template <> struct Mfma<float> {
  typedef float v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 mma(float a, float b, v4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int arow(int x) { return ((x & 3) >> 1) * 8 + (x >> 2) * 2 + (x & 1); }
};

// Which A row and which k a lane feeds to the MFMAs.  Lane (r, g) = (lane % 16,
// lane / 16) supplies, to MFMA tile i at k-step q of a stage, element
//   row(i, r) = 32*(i/2) + 2*arow(r) + i%2
// of the wave's slice of A at k = kq(q) + kg(g), and reads the matching B
// element from LDS row k.  Rows come in adjacent pairs (tiles 2h, 2h+1), so
// one 16-byte load fills two MFMA operands when A is M-contiguous.  When A is
// K-contiguous (PAIR_K) k comes in adjacent pairs instead (steps 2p, 2p+1):
//   kq(q) = 8*(q/2) + q%2, kg(g) = 2*g;  otherwise kq(q) = 4*q, kg(g) = g,
// which keeps every k-step on four consecutive k (a step wholly past the end
// of K is skipped).  After the MFMAs lane (r, g) holds, for column r of each
// 16-column tile j, P = 16 / sizeof(T) consecutive rows per unit u (U = 8 / P
// units per h):
//   rows 32h + 4P*u + P*g + p, p < P,  element p in acc[2h + p%2][j][u*P/2 + p/2],
// so lanes g = 0..3 of a column cover rows 32h + 4P*u .. + 4P - 1 together.
__device__ __forceinline__ int a_row(int i, int arow) { return 32 * (i >> 1) + 2 * arow + (i & 1); }
template <int MODE> __device__ __forceinline__ int kq_of(int q);
template <int MODE> __device__ __forceinline__ int kg_of(int g);

constexpr uint32_t OOB_OFFSET = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;   // raw (untyped) buffer access on CDNA

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7fffffff, BUF_WORD3);
}

// Every load is (per-lane byte offset, wave-uniform byte offset): the uniform
// part goes in the instruction's scalar offset, so one vector register per
// operand carries the lane's address.  An element outside the operand gets
// the per-lane offset 2^31, past the resource's 2^31 - 1 byte range, and the
// hardware returns zero for it without touching memory.  Valid elements are at
// byte offsets below 2^31 (leading dimensions are below 2^21).
template <typename T> struct Ld;
template <> struct Ld<double> {
  typedef double v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ double one(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, v, s, 0));
  }
  static __device__ __forceinline__ v2 two(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
    return __builtin_bit_cast(v2, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0));
  }
};
template <> struct Ld<float> {
  typedef float v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float one(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, v, s, 0));
  }
  static __device__ __forceinline__ v2 two(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
    return __builtin_bit_cast(v2, __builtin_amdgcn_raw_buffer_load_b64(r, v, s, 0));
  }
};

__device__ __forceinline__ uint32_t lane_off(bool ok, uint32_t v) { return ok ? v : OOB_OFFSET; }

// Load modes (tlr_desc.h): LOAD_PAIR_M (A M-contiguous, one 16-byte load gives
// rows 2h and 2h+1 of one k), LOAD_PAIR_K (A K-contiguous, one load gives
// k-steps 2p and 2p+1 of one row) and LOAD_SINGLE (one element per load).  The
// pair modes move B two elements per load as well.  The host only gives a
// pair mode to a task whose operands allow it: pair-aligned bases and
// offsets, even leading dimensions and an even extent along every paired
// index, so that a pair lies wholly inside an operand or wholly outside it.
constexpr int SINGLE = LOAD_SINGLE, PAIR_M = LOAD_PAIR_M, PAIR_K = LOAD_PAIR_K;

template <int MODE> __device__ __forceinline__ int kq_of(int q) {
  return MODE == PAIR_K ? 8 * (q >> 1) + (q & 1) : 4 * q;
}
template <int MODE> __device__ __forceinline__ int kg_of(int g) { return MODE == PAIR_K ? 2 * g : g; }

template <typename T>
struct SegCtx {
  const T *aw;          // A at the wave's first row
  const T *b;           // B at (k = 0, n = n0)
  int32_t lda, ldb, K;
  bool a_xc, b_xc;      // A: M contiguous; B: N contiguous
  int mrem, nrem;       // rows of the wave's slice / columns of the block inside the operand
  int32_t sr, sk;       // element strides of A along a row step and a k step
  uint32_t a_lane;      // byte offset of the lane's (row 2*arow, k 2*g) in the slice
  int row2, gk;         // 2*arow and the lane's k offset kg(g)
};

// A fragments needed after k-step q of a stage are loaded for the stage that
// starts at k0.  Row and k split into a lane part (2*arow, 2*g) and a
// wave-uniform part (ri, qk), and so does the bounds check.
template <typename T, int MODE>
__device__ __forceinline__ void load_a(const SegCtx<T> &c, int k0, int q, T (&fa)[MI][4]) {
  const int krem = c.K - k0;
  const __amdgpu_buffer_rsrc_t rs = rsrc(c.a_xc ? c.aw + (int64_t)k0 * c.lda : c.aw + k0);
  constexpr uint32_t SZ = sizeof(T);
  if (MODE == PAIR_M) {
    const int qk = kq_of<MODE>(q);
    const bool kok = c.gk < krem - qk;
#pragma unroll
    for (int h = 0; h < MI / 2; ++h) {
      const int ri = 32 * h;
      const bool ok = kok && c.row2 < c.mrem - ri;
      const typename Ld<T>::v2 v = Ld<T>::two(rs, lane_off(ok, c.a_lane), (uint32_t)(ri * c.sr + qk * c.sk) * SZ);
      fa[2 * h][q] = v.x;
      fa[2 * h + 1][q] = v.y;
    }
  } else if (MODE == PAIR_K) {
    if (q & 1) {
      const int qk = kq_of<MODE>(q - 1);
      const bool kok = c.gk < krem - qk;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int ri = 32 * (i >> 1) + (i & 1);
        const bool ok = kok && c.row2 < c.mrem - ri;
        const typename Ld<T>::v2 v = Ld<T>::two(rs, lane_off(ok, c.a_lane), (uint32_t)(ri * c.sr + qk * c.sk) * SZ);
        fa[i][q - 1] = v.x;
        fa[i][q] = v.y;
      }
    }
  } else {
    const int qk = kq_of<MODE>(q);
    const bool kok = c.gk < krem - qk;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int ri = 32 * (i >> 1) + (i & 1);
      const bool ok = kok && c.row2 < c.mrem - ri;
      fa[i][q] = Ld<T>::one(rs, lane_off(ok, c.a_lane), (uint32_t)(ri * c.sr + qk * c.sk) * SZ);
    }
  }
}

// Which B elements one thread moves per stage.  Single mode: EPT elements
// (x + p*dx, k + p*dk) (x = n inside the block); pair mode: EPT/2 pairs, the
// second element of a pair one further along the contiguous index (in LDS +1
// along n, +LDS_B along k).  Entry p sits at byte offset lane + p*step of the
// stage's resource and at LDS index lds + p*lds_step.
struct BMap {
  uint32_t lane, step;
  int32_t x, dx, k, dk;
  int32_t lds, lds_step, lds2;
};

template <int MODE, int NJ, typename T>
__device__ __forceinline__ BMap b_map(bool xc, int32_t ld, int tid) {
  constexpr int KBN = Blk<NJ>::KBN, LDS_B = Blk<NJ>::LDS_B;
  BMap m;
  int32_t lin, st;
  if (MODE == SINGLE) {
    if (xc) {   // lanes walk n
      m.x = tid % KBN; m.dx = 0; m.k = tid / KBN; m.dk = NT / KBN;
      lin = m.x + m.k * ld; st = m.dk * ld;
    } else {    // lanes walk k
      m.k = tid & 15; m.dk = 0; m.x = tid >> 4; m.dx = NT / 16;
      lin = m.k + m.x * ld; st = m.dx * ld;
    }
    m.lds2 = 0;
  } else {
    if (xc) {   // pairs along n: KBN / 2 pairs cover a k-row
      m.x = 2 * (tid % (KBN / 2)); m.dx = 0; m.k = tid / (KBN / 2); m.dk = NT / (KBN / 2);
      lin = m.x + m.k * ld; st = m.dk * ld;
      m.lds2 = 1;
    } else {    // pairs along k: 8 pairs cover a column
      m.k = 2 * (tid & 7); m.dk = 0; m.x = tid >> 3; m.dx = NT / 8;
      lin = m.k + m.x * ld; st = m.dx * ld;
      m.lds2 = LDS_B;
    }
  }
  m.lane = (uint32_t)lin * (uint32_t)sizeof(T);
  m.step = (uint32_t)st * (uint32_t)sizeof(T);
  m.lds = m.k * LDS_B + m.x;
  m.lds_step = m.dk * LDS_B + m.dx;
  return m;
}

template <typename T, int MODE, int NJ, int EPT = Blk<NJ>::EPT>
__device__ __forceinline__ void load_b(const SegCtx<T> &c, const BMap &m, int k0, T (&rb)[EPT]) {
  const int krem = c.K - k0;
  const __amdgpu_buffer_rsrc_t rs = rsrc(c.b_xc ? c.b + (int64_t)k0 * c.ldb : c.b + k0);
  if (MODE == SINGLE) {
#pragma unroll
    for (int p = 0; p < EPT; ++p) {
      const bool ok = m.x < c.nrem - p * m.dx && m.k < krem - p * m.dk;
      rb[p] = Ld<T>::one(rs, lane_off(ok, m.lane), p * m.step);
    }
  } else {
#pragma unroll
    for (int p = 0; p < EPT / 2; ++p) {
      const bool ok = m.x < c.nrem - p * m.dx && m.k < krem - p * m.dk;
      const typename Ld<T>::v2 v = Ld<T>::two(rs, lane_off(ok, m.lane), p * m.step);
      rb[2 * p] = v.x;
      rb[2 * p + 1] = v.y;
    }
  }
}

template <int MODE, int NJ, typename T, int EPT = Blk<NJ>::EPT>
__device__ __forceinline__ void store_b(const BMap &m, const T (&rb)[EPT], T *Bs) {
  if (MODE == SINGLE) {
#pragma unroll
    for (int p = 0; p < EPT; ++p) Bs[m.lds + p * m.lds_step] = rb[p];
  } else {
#pragma unroll
    for (int p = 0; p < EPT / 2; ++p) {
      T *q = Bs + m.lds + p * m.lds_step;
      q[0] = rb[2 * p];
      q[m.lds2] = rb[2 * p + 1];
    }
  }
}

// One K segment.  Pipeline of a stage st (16 k, four k-steps q):
//   k-step q:  LDS fragments of step q+1 are read while step q's MFMAs run
//              (fragments double-buffered in registers), and A for stage
//              st+1 is loaded into the registers step q just released;
//   after q=1: the B tile of stage st+1 (loaded from global memory one
//              stage earlier) goes to LDS buffer (st+1)%3, one barrier, and
//              the global loads of stage st+2's B tile are issued;
//   k-step 3:  reads stage st+1's first fragments from the new buffer.
// Three LDS buffers make one barrier per stage enough: buffer (st+1)%3 was
// last read in stage st-2, before every wave passed stage st-1's barrier.
// The barrier sits mid-stage, with two k-steps of MFMAs (and their operands)
// still to issue behind it, so a wave that waits there loses no fragment
// latency.  B loads past the end of K come back as zeros and are never used.
template <typename T, int MODE, int NJ>
__device__ __forceinline__ void run_segment(SegCtx<T> c, int tid, int arow, int g, int r, int wn,
                                            T (*Bs)[KBK * Blk<NJ>::LDS_B], typename Mfma<T>::v4 (&acc)[MI][NJ]) {
  constexpr int LDS_B = Blk<NJ>::LDS_B, EPT = Blk<NJ>::EPT;
  const int nst = (c.K + KBK - 1) / KBK;
  if (nst <= 0) return;
  c.gk = kg_of<MODE>(g);
  c.a_lane = (uint32_t)(c.row2 * c.sr + c.gk * c.sk) * (uint32_t)sizeof(T);
  const int klast = c.K - (nst - 1) * KBK;   // valid k of the last stage
  const BMap bm = b_map<MODE, NJ, T>(c.b_xc, c.ldb, tid);
  T fa[MI][4];
  T rb[EPT];
  T bf[2][NJ];
  auto read_b = [&](const T *Bb, int q, T (&b)[NJ]) {
    const T *br = Bb + (kq_of<MODE>(q) + kg_of<MODE>(g)) * LDS_B + wn + r;
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = br[16 * j];
  };
#pragma unroll
  for (int q = 0; q < 4; ++q) load_a<T, MODE>(c, 0, q, fa);
  load_b<T, MODE, NJ>(c, bm, 0, rb);
  __syncthreads();   // the previous segment's last reads of every buffer are done
  store_b<MODE, NJ>(bm, rb, Bs[0]);
  load_b<T, MODE, NJ>(c, bm, KBK, rb);   // stage 1 (zeros when there is none)
  __syncthreads();
  read_b(Bs[0], 0, bf[0]);
  // The last stage is peeled so that the loop body holds no conditional loads
  // (a load under a branch makes the compiler wait for every outstanding load
  // at the join).
  int cur = 0;   // LDS buffer of stage st: st % 3
  auto stage = [&](int st, auto more_tag) {
    constexpr bool MORE = decltype(more_tag)::value;
    const int k1 = (st + 1) * KBK;
    const int nxt = cur == 2 ? 0 : cur + 1;
    const T *Bb = Bs[cur];
#pragma unroll
    for (int q = 0; q < KBK / 4; ++q) {
      if (!MORE && kq_of<MODE>(q) >= klast) continue;   // every k of this step is past K
      T(&b)[NJ] = bf[q & 1];
      if (q + 1 < KBK / 4) {
        if (MORE || kq_of<MODE>(q + 1) < klast) read_b(Bb, q + 1, bf[(q + 1) & 1]);
      } else if (MORE) {
        read_b(Bs[nxt], 0, bf[0]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = Mfma<T>::mma(fa[i][q], b[j], acc[i][j]);
      if (MORE) {
        // Interleave the next k-step's B fragment reads with this k-step's
        // MFMAs: one LDS read, then MI MFMAs, from the start of the k-step.
        // Left to itself the compiler issued the reads after all but the
        // last MFMA, and the next k-step's first MFMAs waited for them;
        // interleaved, the final update and the dense GEMM ran 2% faster.
        // (sched_group_barrier masks: 0x100 LDS reads, 0x008 MFMAs.)
#pragma unroll
        for (int k = 0; k < NJ; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, MI, 0);
        }
      }
      if (MORE) load_a<T, MODE>(c, k1, q, fa);
      if (MORE && q == 1) {
        store_b<MODE, NJ>(bm, rb, Bs[nxt]);
        __syncthreads();
        load_b<T, MODE, NJ>(c, bm, k1 + KBK, rb);
      }
    }
    cur = nxt;
  };
  for (int st = 0; st + 1 < nst; ++st) stage(st, std::true_type{});
  stage(nst - 1, std::false_type{});
}

template <typename T, int MODE0, int NJ>
__device__ __forceinline__ void gemm_block(const DevTask &t, int m0, int n0, const int64_t *coltab,
                                           const Bases &bases, T alpha, T beta, T cscale) {
  typedef typename Mfma<T>::v4 v4;
  __shared__ T Bs[3][KBK * Blk<NJ>::LDS_B];
  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: readfirstlane tells the compiler
  // so, which keeps operand addresses and buffer resources in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave * WM, wn = 0;
  const int r = lane & 15, g = lane >> 4;
  const int arow = Mfma<T>::arow(r);
  const int M = t.M, N = t.N;

  // C <- alpha*(acc + (beta/alpha)*C): when the host found beta/alpha finite the
  // old C is read into the accumulators before the K loop (its latency hides
  // behind the first loads) and the epilogue only stores.
  T *C = static_cast<T *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;
  const bool fin = t.final_ != 0;
  const bool vec = (t.flags & TASK_VEC) && (reinterpret_cast<uintptr_t>(C) % 16 == 0);
  const bool preload = fin && cscale != T(0);
  const bool rd = fin && beta != T(0) && !preload;
  // C moves in 16-byte units of P rows (the lane layout above)
  constexpr int P = 16 / (int)sizeof(T), U = 8 / P;
  typedef T vp __attribute__((ext_vector_type(P)));
  // A wave whose 32 x 128 slice lies wholly inside the task moves C on
  // branch-free paths, so that all of a lane's accesses go out back to back.
  const bool full = vec && m0 + wm + 32 * (MI / 2) <= M && n0 + wn + 16 * NJ <= N;
  v4 acc[MI][NJ];
  if (preload && full) {
    int64_t cols[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn + 16 * j + r;
      cols[j] = t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n];
    }
    vp x[NJ][MI / 2][U];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int h = 0; h < MI / 2; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u)
          x[j][h][u] = *reinterpret_cast<const vp *>(C + cols[j] + (m0 + wm + 32 * h + 4 * P * u + P * g));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int h = 0; h < MI / 2; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < P; ++e) acc[2 * h + (e & 1)][j][u * (P / 2) + (e >> 1)] = cscale * x[j][h][u][e];
  } else
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + r;
    const int64_t col = (!preload || n >= N) ? 0 : (t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n]);
    const T *cp = C + col;
#pragma unroll
    for (int h = 0; h < MI / 2; ++h) {
      acc[2 * h][j] = v4{0, 0, 0, 0};
      acc[2 * h + 1][j] = v4{0, 0, 0, 0};
      if (!preload || n >= N) continue;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int m = m0 + wm + 32 * h + 4 * P * u + P * g;
        if (vec && m + P - 1 < M) {
          const vp x = cscale * *reinterpret_cast<const vp *>(cp + m);
#pragma unroll
          for (int e = 0; e < P; ++e) acc[2 * h + (e & 1)][j][u * (P / 2) + (e >> 1)] = x[e];
        } else {
#pragma unroll
          for (int e = 0; e < P; ++e)
            if (m + e < M) acc[2 * h + (e & 1)][j][u * (P / 2) + (e >> 1)] = cscale * cp[m + e];
        }
      }
    }
  }

  // t lives in global (or kernel-argument) memory: the segment descriptor is
  // read with scalar loads per iteration instead of being held in registers
  const int nseg = t.nseg;
  auto setup = [&](const DevSeg &d, SegCtx<T> &c) {
    const T *a = static_cast<const T *>(bases.p[d.a.base]) + d.a.off;
    const T *b = static_cast<const T *>(bases.p[d.b.base]) + d.b.off;
    c.lda = d.a.ld;
    c.ldb = d.b.ld;
    c.K = d.K;
    c.a_xc = d.a.trans == 0;
    c.b_xc = d.b.trans == 1;
    c.aw = c.a_xc ? a + (m0 + wm) : a + (int64_t)(m0 + wm) * c.lda;
    c.b = c.b_xc ? b + n0 : b + (int64_t)n0 * c.ldb;
    c.mrem = M - m0 - wm;
    c.nrem = N - n0;
    c.sr = c.a_xc ? 1 : c.lda;
    c.sk = c.a_xc ? c.lda : 1;
    c.row2 = 2 * arow;
    c.a_lane = 0;   // set per load mode in run_segment
  };
  if (nseg > 0) { SegCtx<T> c; setup(t.seg[0], c); run_segment<T, MODE0, NJ>(c, tid, arow, g, r, wn, Bs, acc); }
  if (nseg > 1) { SegCtx<T> c; setup(t.seg[1], c); run_segment<T, SINGLE, NJ>(c, tid, arow, g, r, wn, Bs, acc); }

  // Epilogue: one 16-byte unit per lane, column and u (when the column start is
  // 16-byte aligned).  Every column offset is read before the first store:
  // the memory counter that a wait for a column-map load uses also counts the
  // stores issued before it, so a map lookup between stores would wait for
  // all of them to complete.
  int64_t ocol[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + r;
    ocol[j] = n >= N ? 0 : (t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n]);
  }
  // The stores keep their per-unit checks even for a slice wholly inside the
  // task: a branch-free run of 32 back-to-back stores per wave measured slower,
  // since the burst holds up the co-resident workgroup's operand loads in the
  // CU's shared memory pipeline.
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + r;
    if (n >= N) continue;
    T *cp = C + ocol[j];
#pragma unroll
    for (int h = 0; h < MI / 2; ++h) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        vp x;
#pragma unroll
        for (int e = 0; e < P; ++e) x[e] = acc[2 * h + (e & 1)][j][u * (P / 2) + (e >> 1)];
        if (fin) x = alpha * x;
        const int m = m0 + wm + 32 * h + 4 * P * u + P * g;
        if (vec && m + P - 1 < M) {
          vp *q = reinterpret_cast<vp *>(cp + m);
          if (rd) x += beta * *q;
          *q = x;
        } else {
#pragma unroll
          for (int e = 0; e < P; ++e) {
            if (m + e < M) {
              T y = x[e];
              if (rd) y += beta * cp[m + e];
              cp[m + e] = y;
            }
          }
        }
      }
    }
  }
}

// MODE: load mode of the first segment of every task in the table (the
// table is split by mode on the host); a second segment, the small diagonal
// term of a tile, always runs in single-element mode.
template <typename T, int STAGE, int MODE, int NJ>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Blk<NJ>::WAVES_PER_EU)))
void grouped_gemm_kernel(const DevTask *__restrict__ tasks, const DevTile *__restrict__ tiles,
                         const int64_t *__restrict__ coltab, Bases bases, T alpha, T beta, T cscale) {
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask &t = tasks[e.task];
  const bool fin = t.final_ != 0;
  gemm_block<T, MODE, NJ>(t, e.m0, e.n0, coltab, bases, fin ? alpha : T(1), fin ? beta : T(0), fin ? cscale : T(0));
}

// Single task given by value; blockIdx.x walks the output blocks so that each
// XCD (workgroups are dealt to the 8 XCDs round-robin) takes a contiguous run
// of block indices, ordered in bands of 8 block rows for L2 reuse.
template <typename T, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
void single_gemm_kernel(DevTask t, Bases bases, T alpha, T beta, T cscale, int mt, int nt, int per) {
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * per + (bid >> 3);
  if (logical >= mt * nt) return;
  const int band = 8;
  const int group = logical / (band * nt);
  const int first_m = group * band;
  const int rows = min(band, mt - first_m);
  const int in = logical - group * band * nt;
  const int mtile = first_m + in % rows;
  const int ntile = in / rows;
  gemm_block<T, MODE, 8>(t, mtile * KBM, ntile * Blk<8>::KBN, nullptr, bases, alpha, beta, cscale);
}

// One task per tile of a regular grid (TileGemm): workgroup x = (tile, row
// block); the tile's task (N <= 128, one block column of 16 NJ columns) is
// built from the tile's extents.  C = A B, no alpha / beta.
template <typename T, int MODE, int NJ>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Blk<NJ>::WAVES_PER_EU)))
void tile_gemm_kernel(TileGemm g, Bases bases, int mb_per_tile) {
  const int t = blockIdx.x / mb_per_tile, mb = blockIdx.x - t * mb_per_tile;
  if (t >= g.qr * g.qc) return;
  const int i = t % g.qr, j = t / g.qr;
  if (g.skip_diag && i == j) return;
  const int64_t ro = (int64_t)i * g.b, co = (int64_t)j * g.b;
  const int si = (int)min<int64_t>(g.b, g.rows - ro), sj = (int)min<int64_t>(g.b, g.cols - co);
  const int M = g.m_sel == 0 ? si : (g.m_sel == 1 ? sj : g.n_fixed);
  const int K = g.k_sel == 0 ? si : (g.k_sel == 1 ? sj : g.n_fixed);
  if (mb * KBM >= M) return;
  auto opnd = [&](const TileAddr &x) {
    DevOperand o;
    o.off = x.off + ro * x.f_ro + co * x.f_co + (int64_t)t * x.f_t;
    o.ld = x.ld;
    o.base = x.base;
    o.trans = x.trans;
    o.flags = 0;
    return o;
  };
  DevTask task;
  task.M = M;
  task.N = g.n;
  task.c_off = g.c.off + ro * g.c.f_ro + co * g.c.f_co + (int64_t)t * g.c.f_t;
  task.ctab = -1;
  task.ldc = g.c.ld;
  task.c_base = g.c.base;
  task.final_ = 0;
  task.nseg = K > 0 ? 1 : 0;
  constexpr int VEC = 16 / (int)sizeof(T);
  task.flags = (task.c_off % VEC == 0 && task.ldc % VEC == 0) ? TASK_VEC : 0;
  task.seg[0].a = opnd(g.a);
  task.seg[0].b = opnd(g.bop);
  task.seg[0].K = K;
  task.seg[0].pad = 0;
  gemm_block<T, MODE, NJ>(task, mb * KBM, 0, nullptr, bases, T(1), T(0), T(0));
}

// Strip blocks for the right/left product (stage 2).  Its tasks have one K
// segment of at most one stage (ranks up to 16) and store C = acc through the
// column map, so their time goes to the stores; a 128 x 128 block spends about
// as long fetching its few operands as it then spends storing.  A strip block
// covers 128 rows and STRIP_W columns: it loads its A rows into registers and
// the B operand and the column offsets of all STRIP_W columns into LDS once,
// then runs 128-column chunks back to back, each a few MFMAs and then the
// chunk's stores, with no barrier between chunks, so that the stores of one
// wave run while the MFMAs of the others do.  B is N-contiguous (the coupling
// matrix as the planner stores it for this product), which keeps every byte
// offset of the fill below 2^31 (k < 16, leading dimensions below 2^21).
constexpr int SPAD = 17;                 // odd LDS row stride, as for the B tiles above
constexpr int LDS_S = STRIP_W + SPAD;

template <typename T, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
void strip_gemm_kernel(const DevTask *__restrict__ tasks, const DevTile *__restrict__ tiles,
                       const int64_t *__restrict__ coltab, Bases bases) {
  typedef typename Mfma<T>::v4 v4;
  constexpr int NJ = 8, KBN = Blk<NJ>::KBN;
  static_assert(STRIP_W == 2 * NT && STRIP_W % KBN == 0, "strip fill: two columns per thread");
  __shared__ T Bs[KBK * LDS_S];
  __shared__ int64_t cols[STRIP_W];
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask &t = tasks[e.task];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave * WM;
  const int r = lane & 15, g = lane >> 4;
  const int arow = Mfma<T>::arow(r);
  const int M = t.M, m0 = e.m0, n0 = e.n0;
  const int nrem = min(t.N - n0, STRIP_W);
  const int K = t.nseg > 0 ? t.seg[0].K : 0;   // a task without a segment stores zeros
  const DevSeg &d = t.seg[0];
  T *C = static_cast<T *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;

  T fa[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) fa[i][q] = T(0);
  if (K > 0) {
    const T *a = static_cast<const T *>(bases.p[d.a.base]) + d.a.off;
    const T *b = static_cast<const T *>(bases.p[d.b.base]) + d.b.off + n0;
    SegCtx<T> c;
    c.lda = d.a.ld;
    c.ldb = d.b.ld;
    c.K = K;
    c.a_xc = d.a.trans == 0;
    c.b_xc = true;
    c.aw = c.a_xc ? a + (m0 + wm) : a + (int64_t)(m0 + wm) * c.lda;
    c.b = b;
    c.mrem = M - m0 - wm;
    c.nrem = nrem;
    c.sr = c.a_xc ? 1 : c.lda;
    c.sk = c.a_xc ? c.lda : 1;
    c.row2 = 2 * arow;
    c.gk = kg_of<MODE>(g);
    c.a_lane = (uint32_t)(c.row2 * c.sr + c.gk * c.sk) * (uint32_t)sizeof(T);
#pragma unroll
    for (int q = 0; q < 4; ++q) load_a<T, MODE>(c, 0, q, fa);
    // B (K x nrem, N contiguous) -> LDS rows k, zeros past K and past nrem
    const __amdgpu_buffer_rsrc_t rs = rsrc(b);
    if (MODE != SINGLE) {   // pairs along n: a pair lies inside B or ends in its padding
      const int n = 2 * tid;
#pragma unroll
      for (int k = 0; k < KBK; ++k) {
        const bool ok = k < K && n < nrem;
        const typename Ld<T>::v2 v = Ld<T>::two(rs, lane_off(ok, (uint32_t)(k * c.ldb + n) * (uint32_t)sizeof(T)), 0);
        Bs[k * LDS_S + n] = v.x;
        Bs[k * LDS_S + n + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int k = 0; k < KBK; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int n = tid + NT * h;
          const bool ok = k < K && n < nrem;
          Bs[k * LDS_S + n] = Ld<T>::one(rs, lane_off(ok, (uint32_t)(k * c.ldb + n) * (uint32_t)sizeof(T)), 0);
        }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = tid + NT * h;
    cols[n] = n >= nrem ? 0 : (t.ctab < 0 ? (int64_t)(n0 + n) * t.ldc : coltab[t.ctab + n0 + n]);
  }
  __syncthreads();

  const bool vec = (t.flags & TASK_VEC) && (reinterpret_cast<uintptr_t>(C) % 16 == 0);
  constexpr int P = 16 / (int)sizeof(T), U = 8 / P;
  typedef T vp __attribute__((ext_vector_type(P)));
  const int nch = (nrem + KBN - 1) / KBN;
  for (int ch = 0; ch < nch; ++ch) {
    v4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = v4{0, 0, 0, 0};
    if (K > 0) {
#pragma unroll
      for (int q = 0; q < KBK / 4; ++q) {
        if (kq_of<MODE>(q) >= K) continue;   // every k of this step is past K
        const T *br = Bs + (kq_of<MODE>(q) + kg_of<MODE>(g)) * LDS_S + ch * KBN + r;
        T bq[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) bq[j] = br[16 * j];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = Mfma<T>::mma(fa[i][q], bq[j], acc[i][j]);
      }
    }
    // stores: the lane layout of gemm_block's epilogue
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = ch * KBN + 16 * j + r;
      if (n >= nrem) continue;
      T *cp = C + cols[n];
#pragma unroll
      for (int h = 0; h < MI / 2; ++h) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          vp x;
#pragma unroll
          for (int q = 0; q < P; ++q) x[q] = acc[2 * h + (q & 1)][j][u * (P / 2) + (q >> 1)];
          const int m = m0 + wm + 32 * h + 4 * P * u + P * g;
          if (vec && m + P - 1 < M) {
            *reinterpret_cast<vp *>(cp + m) = x;
          } else {
#pragma unroll
            for (int q = 0; q < P; ++q)
              if (m + q < M) cp[m + q] = x[q];
          }
        }
      }
    }
  }
}

template <typename T>
__global__ void scale_kernel(T *C, int64_t m, int64_t n, int64_t ldc, T beta) {
  const int64_t total = m * n;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = idx / m, r = idx - c * m;
    T *p = C + r + c * ldc;
    *p = beta == T(0) ? T(0) : beta * *p;
  }
}

// beta/alpha when C can be pre-scaled into the accumulators, else 0 (then the
// epilogue reads C and adds beta*C after scaling by alpha).  The pre-scaled
// form computes alpha*((beta/alpha)*C + sum), so it is used only when
// |beta/alpha| <= 1 (the scaled C cannot overflow where C does not) and
// |beta/alpha| is a normal number of T (a subnormal ratio would drop digits
// of the beta*C term).
template <typename T>
T preload_scale(double alpha, double beta) {
  if (beta == 0.0 || alpha == 0.0) return T(0);
  const double r = beta / alpha, a = r < 0 ? -r : r;
  const double tiny = sizeof(T) == 8 ? 2.2250738585072014e-308 : 1.1754943508222875e-38;
  return (a <= 1.0 && a >= tiny) ? T(r) : T(0);
}

template <typename T, int STAGE, int NJ>
void launch_grouped_s(int mode, dim3 grid, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                      const int64_t *coltab, const Bases &bases, T a, T b, T c) {
  const dim3 block(NT);
  if (mode == LOAD_PAIR_M)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, STAGE, LOAD_PAIR_M, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else if (mode == LOAD_PAIR_K)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, STAGE, LOAD_PAIR_K, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<T, STAGE, LOAD_SINGLE, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
}

template <typename T, int NJ>
void launch_grouped_w(int stage, int mode, dim3 grid, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                      const int64_t *coltab, const Bases &bases, T a, T b, T c) {
  if (stage == 1)
    launch_grouped_s<T, 1, NJ>(mode, grid, s, tasks, tiles, coltab, bases, a, b, c);
  else if (stage == 2)
    launch_grouped_s<T, 2, NJ>(mode, grid, s, tasks, tiles, coltab, bases, a, b, c);
  else if (stage == 3)
    launch_grouped_s<T, 3, NJ>(mode, grid, s, tasks, tiles, coltab, bases, a, b, c);
  else
    launch_grouped_s<T, STAGE_SIDE, NJ>(mode, grid, s, tasks, tiles, coltab, bases, a, b, c);
}

template <typename T>
void launch_strip_t(int mode, unsigned n, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                    const int64_t *coltab, const Bases &bases) {
  const dim3 grid(n), block(NT);
  if (mode == LOAD_PAIR_M)
    hipLaunchKernelGGL((strip_gemm_kernel<T, LOAD_PAIR_M>), grid, block, 0, s, tasks, tiles, coltab, bases);
  else if (mode == LOAD_PAIR_K)
    hipLaunchKernelGGL((strip_gemm_kernel<T, LOAD_PAIR_K>), grid, block, 0, s, tasks, tiles, coltab, bases);
  else
    hipLaunchKernelGGL((strip_gemm_kernel<T, LOAD_SINGLE>), grid, block, 0, s, tasks, tiles, coltab, bases);
}

template <typename T>
void launch_grouped_t(int stage, int mode, int bn, unsigned n, hipStream_t s, const DevTask *tasks,
                      const DevTile *tiles, const int64_t *coltab, const Bases &bases, double alpha, double beta) {
  const T a = (T)alpha, b = (T)beta, c = preload_scale<T>(alpha, beta);
  const dim3 grid(n);
  if (bn == STRIP_W)
    launch_strip_t<T>(mode, n, s, tasks, tiles, coltab, bases);
  else if (bn == Blk<4>::KBN)
    launch_grouped_w<T, 4>(stage, mode, grid, s, tasks, tiles, coltab, bases, a, b, c);
  else
    launch_grouped_w<T, 8>(stage, mode, grid, s, tasks, tiles, coltab, bases, a, b, c);
}

template <typename T>
void launch_single_t(int mode, unsigned n, hipStream_t s, const DevTask &task, const Bases &bases, double alpha,
                     double beta, int mt, int nt, int per) {
  const T a = (T)alpha, b = (T)beta, c = preload_scale<T>(alpha, beta);
  const dim3 grid(n), block(NT);
  if (mode == LOAD_PAIR_M)
    hipLaunchKernelGGL((single_gemm_kernel<T, LOAD_PAIR_M>), grid, block, 0, s, task, bases, a, b, c, mt, nt, per);
  else if (mode == LOAD_PAIR_K)
    hipLaunchKernelGGL((single_gemm_kernel<T, LOAD_PAIR_K>), grid, block, 0, s, task, bases, a, b, c, mt, nt, per);
  else
    hipLaunchKernelGGL((single_gemm_kernel<T, LOAD_SINGLE>), grid, block, 0, s, task, bases, a, b, c, mt, nt, per);
}

}  // namespace

int launch_grouped(tlr_dtype dt, int stage, int mode, int bn, const DevTask *tasks, const DevTile *tiles,
                   int64_t n_tiles, const int64_t *coltab, const Bases &bases, double alpha, double beta,
                   void *stream) {
  if (dt == TLR_F16 || dt == TLR_BF16)
    return launch_grouped16(dt, stage, bn, tasks, tiles, n_tiles, coltab, bases, alpha, beta, stream);
  if (n_tiles <= 0) return 0;
  if (bn != Blk<4>::KBN && bn != Blk<8>::KBN && !(bn == STRIP_W && stage == 2)) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F64)
    launch_grouped_t<double>(stage, mode, bn, (unsigned)n_tiles, s, tasks, tiles, coltab, bases, alpha, beta);
  else
    launch_grouped_t<float>(stage, mode, bn, (unsigned)n_tiles, s, tasks, tiles, coltab, bases, alpha, beta);
  return (int)hipGetLastError();
}

int launch_single(tlr_dtype dt, int mode, const DevTask &task, const Bases &bases, double alpha, double beta,
                  void *stream) {
  const int mt = (task.M + KBM - 1) / KBM, nt = (task.N + Blk<8>::KBN - 1) / Blk<8>::KBN;
  if (mt == 0 || nt == 0) return 0;
  const int64_t n = (int64_t)mt * nt;
  const int per = (int)((n + 7) / 8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F64)
    launch_single_t<double>(mode, (unsigned)(per * 8), s, task, bases, alpha, beta, mt, nt, per);
  else
    launch_single_t<float>(mode, (unsigned)(per * 8), s, task, bases, alpha, beta, mt, nt, per);
  return (int)hipGetLastError();
}

int launch_tile_gemm(tlr_dtype dt, int mode, const TileGemm &g, const Bases &bases, void *stream) {
  if (dt != TLR_F64 && dt != TLR_F32) return (int)hipErrorInvalidValue;
  if (g.n <= 0 || g.n > Blk<8>::KBN || g.qr <= 0 || g.qc <= 0) return g.qr <= 0 || g.qc <= 0 ? 0 : (int)hipErrorInvalidValue;
  const int64_t maxm = g.m_sel == 2 ? g.n_fixed : g.b;
  const int mb = (int)((maxm + KBM - 1) / KBM);
  if (mb <= 0) return 0;
  const dim3 grid((unsigned)((int64_t)g.qr * g.qc * mb)), block(NT);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // tiles of at most 64 columns (the sketch width of a TLR output) take
  // 128 x 64 blocks: half the MFMA work of a 128 x 128 block and one more
  // workgroup per CU
#define TLR_TILE_LAUNCH(TT, NJ)                                                                                \
  do {                                                                                                         \
    if (mode == LOAD_PAIR_M)                                                                                   \
      hipLaunchKernelGGL((tile_gemm_kernel<TT, LOAD_PAIR_M, NJ>), grid, block, 0, s, g, bases, mb);            \
    else if (mode == LOAD_PAIR_K)                                                                              \
      hipLaunchKernelGGL((tile_gemm_kernel<TT, LOAD_PAIR_K, NJ>), grid, block, 0, s, g, bases, mb);            \
    else                                                                                                       \
      hipLaunchKernelGGL((tile_gemm_kernel<TT, LOAD_SINGLE, NJ>), grid, block, 0, s, g, bases, mb);            \
  } while (0)
  const bool narrow = g.n <= Blk<4>::KBN;
  if (dt == TLR_F64) {
    if (narrow) TLR_TILE_LAUNCH(double, 4);
    else TLR_TILE_LAUNCH(double, 8);
  } else {
    if (narrow) TLR_TILE_LAUNCH(float, 4);
    else TLR_TILE_LAUNCH(float, 8);
  }
#undef TLR_TILE_LAUNCH
  return (int)hipGetLastError();
}

int launch_scale(tlr_dtype dt, void *C, int64_t m, int64_t n, int64_t ldc, double beta, void *stream) {
  if (dt == TLR_F16 || dt == TLR_BF16) return launch_scale16(dt, C, m, n, ldc, beta, stream);
  if (m <= 0 || n <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = m * n;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  if (dt == TLR_F64)
    hipLaunchKernelGGL(scale_kernel<double>, dim3(blocks), dim3(256), 0, s, static_cast<double *>(C), m, n, ldc, beta);
  else
    hipLaunchKernelGGL(scale_kernel<float>, dim3(blocks), dim3(256), 0, s, static_cast<float *>(C), m, n, ldc,
                       (float)beta);
  return (int)hipGetLastError();
}

}  // namespace tlr
