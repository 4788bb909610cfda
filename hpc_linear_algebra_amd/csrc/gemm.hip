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
// Work split: 256 threads = 4 wave64s in a 2 x 2 arrangement, each wave owns
// a 64 x 64 sub-block = 4 x 4 MFMA tiles of 16 x 16
// (v_mfma_f64_16x16x4_f64 / v_mfma_f32_16x16x4_f32).  K advances in stages of
// BK = 16, staged through LDS and double-buffered: the global loads of stage
// s+1 are in flight while the MFMAs of stage s run.  Register use is held to
// 256 per lane so that two workgroups share a CU: while one waits on memory
// (its first stage, its C update) the other keeps the matrix cores busy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tlr_plan.h"

namespace tlr {

namespace {

constexpr int KBM = 128, KBN = 128, KBK = 16, KPAD = 16, NTHR = 256;
constexpr int LDS_A = KBM + KPAD, LDS_B = KBN + KPAD;

// Lane layout of the 16x16x4 MFMAs (measured on gfx950): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; accumulator element v of lane l is
// D[row][l % 16] with row = 4*(l/16) + v for fp32 but row = l/16 + 4*v for
// fp64.  For fp64 the A fragment is therefore read with its rows permuted by
// arow(x) = 4*(x%4) + x/4, which makes both types leave rows 4*(l/16)+v, i.e.
// four consecutive rows of one column, in lane l.
template <typename T> struct Mfma;
template <> struct Mfma<double> {
  typedef double v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 mma(double a, double b, v4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int arow(int x) { return ((x & 3) << 2) | (x >> 2); }
};
template <> struct Mfma<float> {
  typedef float v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 mma(float a, float b, v4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int arow(int x) { return x; }
};

// Which 8 elements of a 128 x 16 (A) or 16 x 128 (B) stage one thread moves.
// When the 128-long index x (m for A, n for B) is the contiguous one, lanes
// walk x and each thread takes k = k0, k0+2, ...; otherwise lanes walk k and
// each thread takes x = x0, x0+16, ....  Element p sits at intra-tile offset
// lin + p*step of the operand and at LDS index lds + p*lds_step.
struct ThreadMap {
  int32_t lin, step;
  int32_t x, dx, k, dk;
  int32_t lds, lds_step;
};

__device__ __forceinline__ ThreadMap thread_map(bool x_contig, int32_t ld, int tid, int lds_row) {
  ThreadMap t;
  if (x_contig) {
    const int x = tid & 127, k = tid >> 7;
    t.lin = x + k * ld; t.step = 2 * ld;
    t.x = x; t.dx = 0; t.k = k; t.dk = 2;
    t.lds = k * lds_row + x; t.lds_step = 2 * lds_row;
  } else {
    const int k = tid & 15, x = tid >> 4;
    t.lin = k + x * ld; t.step = 16 * ld;
    t.x = x; t.dx = 16; t.k = k; t.dk = 0;
    t.lds = k * lds_row + x; t.lds_step = 16;
  }
  return t;
}

template <typename T>
struct Seg {
  const T *a, *b;
  int32_t lda, ldb, K;
  bool a_xc, b_xc;        // the M (for A) / N (for B) index is the contiguous one
  ThreadMap ma, mb;
};

template <typename T>
__device__ __forceinline__ Seg<T> make_seg(const DevSeg &g, const Bases &bases, int tid) {
  Seg<T> s;
  s.a = static_cast<const T *>(bases.p[g.a.base]) + g.a.off;
  s.b = static_cast<const T *>(bases.p[g.b.base]) + g.b.off;
  s.lda = g.a.ld;
  s.ldb = g.b.ld;
  s.K = g.K;
  s.a_xc = g.a.trans == 0;   // A(m,k) = A[m + k*lda]
  s.b_xc = g.b.trans == 1;   // B(k,n) = B[n + k*ldb]
  s.ma = thread_map(s.a_xc, s.lda, tid, LDS_A);
  s.mb = thread_map(s.b_xc, s.ldb, tid, LDS_B);
  return s;
}

template <typename T>
__device__ __forceinline__ void load_op(const T *base, int64_t x0, int64_t k0, int32_t ld, bool xc, int xrem,
                                        int krem, const ThreadMap &m, T (&r)[8]) {
  const T *p0 = xc ? base + x0 + k0 * ld : base + k0 + x0 * ld;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int x = m.x + p * m.dx, k = m.k + p * m.dk;
    r[p] = (x < xrem && k < krem) ? p0[m.lin + p * m.step] : T(0);
  }
}

template <typename T>
__device__ __forceinline__ void load_stage(const Seg<T> &s, int k0, int m0, int n0, int M, int N,
                                           T (&ra)[8], T (&rb)[8]) {
  const int krem = s.K - k0;
  load_op<T>(s.a, m0, k0, s.lda, s.a_xc, M - m0, krem, s.ma, ra);
  load_op<T>(s.b, n0, k0, s.ldb, s.b_xc, N - n0, krem, s.mb, rb);
}

template <typename T>
__device__ __forceinline__ void store_stage(const Seg<T> &s, const T (&ra)[8], const T (&rb)[8], T *As, T *Bs) {
#pragma unroll
  for (int p = 0; p < 8; ++p) As[s.ma.lds + p * s.ma.lds_step] = ra[p];
#pragma unroll
  for (int p = 0; p < 8; ++p) Bs[s.mb.lds + p * s.mb.lds_step] = rb[p];
}

template <typename T>
__device__ __forceinline__ void gemm_block(const DevTask &t, int m0, int n0, const int64_t *coltab,
                                           const Bases &bases, T alpha, T beta) {
  typedef typename Mfma<T>::v4 v4;
  __shared__ T As[2][KBK * LDS_A];
  __shared__ T Bs[2][KBK * LDS_B];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int arow = Mfma<T>::arow(lane & 15);
  const int M = t.M, N = t.N;

  v4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4{0, 0, 0, 0};

  const int nseg = t.nseg;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {   // constant segment index: no dynamic indexing into the task
    if (sg >= nseg) break;
    const Seg<T> s = make_seg<T>(t.seg[sg], bases, tid);
    const int nst = (s.K + KBK - 1) / KBK;
    T ra[8], rb[8];
    load_stage<T>(s, 0, m0, n0, M, N, ra, rb);
    __syncthreads();   // the previous segment's last reads of buffer 0 are done
    store_stage<T>(s, ra, rb, As[0], Bs[0]);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const bool more = st + 1 < nst;
      if (more) load_stage<T>(s, (st + 1) * KBK, m0, n0, M, N, ra, rb);
      const T *Ab = As[st & 1];
      const T *Bb = Bs[st & 1];
#pragma unroll
      for (int kq = 0; kq < KBK / 4; ++kq) {
        const int kr = kq * 4 + (lane >> 4);
        T a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = Ab[kr * LDS_A + wm + 16 * i + arow];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bb[kr * LDS_B + wn + 16 * j + (lane & 15)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = Mfma<T>::mma(a[i], b[j], acc[i][j]);
      }
      if (more) store_stage<T>(s, ra, rb, As[(st + 1) & 1], Bs[(st + 1) & 1]);
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+v (v = 0..3), column lane%16 of each
  // 16x16 tile; when the column start is 4-element aligned those four rows go
  // out as one vector access.
  T *C = static_cast<T *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;
  const bool fin = t.final_ != 0;
  const bool rd = fin && beta != T(0);
  const bool vec = (t.flags & TASK_VEC) && (reinterpret_cast<uintptr_t>(C) % (4 * sizeof(T)) == 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn + 16 * j + (lane & 15);
    if (n >= N) continue;
    const int64_t col = t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n];
    T *cp = C + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mb = m0 + wm + 16 * i + 4 * (lane >> 4);
      v4 x = acc[i][j];
      if (fin) x = alpha * x;
      if (vec && mb + 3 < M) {
        v4 *vp = reinterpret_cast<v4 *>(cp + mb);
        if (rd) x += beta * *vp;
        *vp = x;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = mb + v;
          if (m < M) {
            T y = x[v];
            if (rd) y += beta * cp[m];
            cp[m] = y;
          }
        }
      }
    }
  }
}

template <typename T, int STAGE>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2)))
void grouped_gemm_kernel(const DevTask *__restrict__ tasks, const DevTile *__restrict__ tiles,
                         const int64_t *__restrict__ coltab, Bases bases, T alpha, T beta) {
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask t = tasks[e.task];
  const bool fin = t.final_ != 0;
  gemm_block<T>(t, e.m0, e.n0, coltab, bases, fin ? alpha : T(1), fin ? beta : T(0));
}

// Single task given by value; blockIdx.x walks the output blocks so that each
// XCD (workgroups are dealt to the 8 XCDs round-robin) takes a contiguous run
// of block indices, ordered in bands of 8 block rows for L2 reuse.
template <typename T>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2)))
void single_gemm_kernel(DevTask t, Bases bases, T alpha, T beta, int mt, int nt, int per) {
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
  gemm_block<T>(t, mtile * KBM, ntile * KBN, nullptr, bases, alpha, beta);
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

template <typename T>
void launch_grouped_t(int stage, dim3 grid, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                      const int64_t *coltab, const Bases &bases, T alpha, T beta) {
  dim3 block(NTHR);
  if (stage == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 1>), grid, block, 0, s, tasks, tiles, coltab, bases, alpha, beta);
  else if (stage == 2)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 2>), grid, block, 0, s, tasks, tiles, coltab, bases, alpha, beta);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 3>), grid, block, 0, s, tasks, tiles, coltab, bases, alpha, beta);
}

}  // namespace

int launch_grouped(tlr_dtype dt, int stage, const DevTask *tasks, const DevTile *tiles, int64_t n_tiles,
                   const int64_t *coltab, const Bases &bases, double alpha, double beta, void *stream) {
  if (n_tiles <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)n_tiles);
  if (dt == TLR_F64)
    launch_grouped_t<double>(stage, grid, s, tasks, tiles, coltab, bases, alpha, beta);
  else
    launch_grouped_t<float>(stage, grid, s, tasks, tiles, coltab, bases, (float)alpha, (float)beta);
  return (int)hipGetLastError();
}

int launch_single(tlr_dtype dt, const DevTask &task, const Bases &bases, double alpha, double beta,
                  void *stream) {
  const int mt = (task.M + KBM - 1) / KBM, nt = (task.N + KBN - 1) / KBN;
  if (mt == 0 || nt == 0) return 0;
  const int64_t n = (int64_t)mt * nt;
  const int per = (int)((n + 7) / 8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)(per * 8)), block(NTHR);
  if (dt == TLR_F64)
    hipLaunchKernelGGL(single_gemm_kernel<double>, grid, block, 0, s, task, bases, alpha, beta, mt, nt, per);
  else
    hipLaunchKernelGGL(single_gemm_kernel<float>, grid, block, 0, s, task, bases, (float)alpha,
                       (float)beta, mt, nt, per);
  return (int)hipGetLastError();
}

int launch_scale(tlr_dtype dt, void *C, int64_t m, int64_t n, int64_t ldc, double beta, void *stream) {
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
