// Grouped, segmented-K MFMA GEMM for gfx950 (CDNA4), fp64 and fp32.
//
// One kernel runs every stage of the TLR product: each workgroup reads one
// entry (task, m0, n0) of a launch's table and computes the 128 x 128 block of
// that task's output, accumulating over the task's K segments, then writes
// C = alpha*acc + beta*C (final update, C read only when beta != 0) or
// C = acc (workspace intermediates), through an affine or indirect column map.
// Layout of the descriptors: tlr_desc.h.
//
// Work split: 256 threads = 4 wave64s in a 2 x 2 arrangement, each wave owns
// a 64 x 64 sub-block = 4 x 4 MFMA tiles of 16 x 16
// (v_mfma_f64_16x16x4_f64 / v_mfma_f32_16x16x4_f32).  K advances in stages of
// BK = 16, staged through LDS and double-buffered: the global loads of stage
// s+1 are in flight while the MFMAs of stage s run.  LDS rows are padded so
// that the four k-rows one MFMA operand fetch touches fall into different
// banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tlr_plan.h"

namespace tlr {

namespace {

constexpr int KBM = 128, KBN = 128, KBK = 16, KPAD = 16, NTHR = 256;

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

struct SegState {
  const void *a, *b;
  int32_t lda, ldb, K;
  uint8_t ta, tb;
};

template <typename T>
__device__ __forceinline__ void load_stage(const SegState &s, int k0, int m0, int n0, int M, int N,
                                           int tid, T (&ra)[8], T (&rb)[8]) {
  const T *A = static_cast<const T *>(s.a);
  const T *B = static_cast<const T *>(s.b);
  if (s.ta == 0) {          // A(m,k) = A[m + k*lda]: lanes walk m
    const int mm = tid & (KBM - 1);
    const int m = m0 + mm;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int k = k0 + (tid >> 7) + 2 * p;
      ra[p] = (m < M && k < s.K) ? A[(int64_t)m + (int64_t)k * s.lda] : T(0);
    }
  } else {                  // A(m,k) = A[k + m*lda]: lanes walk k
    const int k = k0 + (tid & (KBK - 1));
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int m = m0 + (tid >> 4) + 16 * p;
      ra[p] = (m < M && k < s.K) ? A[(int64_t)k + (int64_t)m * s.lda] : T(0);
    }
  }
  if (s.tb == 0) {          // B(k,n) = B[k + n*ldb]: lanes walk k
    const int k = k0 + (tid & (KBK - 1));
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int n = n0 + (tid >> 4) + 16 * p;
      rb[p] = (n < N && k < s.K) ? B[(int64_t)k + (int64_t)n * s.ldb] : T(0);
    }
  } else {                  // B(k,n) = B[n + k*ldb]: lanes walk n
    const int n = n0 + (tid & (KBN - 1));
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int k = k0 + (tid >> 7) + 2 * p;
      rb[p] = (n < N && k < s.K) ? B[(int64_t)n + (int64_t)k * s.ldb] : T(0);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_stage(const SegState &s, int tid, const T (&ra)[8], const T (&rb)[8],
                                            T (*As)[KBM + KPAD], T (*Bs)[KBN + KPAD]) {
  if (s.ta == 0) {
    const int mm = tid & (KBM - 1);
#pragma unroll
    for (int p = 0; p < 8; ++p) As[(tid >> 7) + 2 * p][mm] = ra[p];
  } else {
    const int kk = tid & (KBK - 1);
#pragma unroll
    for (int p = 0; p < 8; ++p) As[kk][(tid >> 4) + 16 * p] = ra[p];
  }
  if (s.tb == 0) {
    const int kk = tid & (KBK - 1);
#pragma unroll
    for (int p = 0; p < 8; ++p) Bs[kk][(tid >> 4) + 16 * p] = rb[p];
  } else {
    const int nn = tid & (KBN - 1);
#pragma unroll
    for (int p = 0; p < 8; ++p) Bs[(tid >> 7) + 2 * p][nn] = rb[p];
  }
}

__device__ __forceinline__ SegState seg_state(const DevSeg &g, const Bases &bases, int es) {
  SegState s;
  s.a = static_cast<const char *>(bases.p[g.a.base]) + g.a.off * es;
  s.b = static_cast<const char *>(bases.p[g.b.base]) + g.b.off * es;
  s.lda = g.a.ld;
  s.ldb = g.b.ld;
  s.K = g.K;
  s.ta = g.a.trans;
  s.tb = g.b.trans;
  return s;
}

template <typename T>
__device__ __forceinline__ void gemm_block(const DevTask &t, int m0, int n0, const int64_t *coltab,
                                           const Bases &bases, T alpha, T beta) {
  typedef typename Mfma<T>::v4 v4;
  __shared__ T As[2][KBK][KBM + KPAD];
  __shared__ T Bs[2][KBK][KBN + KPAD];
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
  SegState s0 = {}, s1 = {};
  int nst0 = 0, nst1 = 0;
  if (nseg > 0) { s0 = seg_state(t.seg[0], bases, (int)sizeof(T)); nst0 = (s0.K + KBK - 1) / KBK; }
  if (nseg > 1) { s1 = seg_state(t.seg[1], bases, (int)sizeof(T)); nst1 = (s1.K + KBK - 1) / KBK; }
  const int total = nst0 + nst1;

  if (total > 0) {
    T ra[8], rb[8];
    load_stage<T>(s0.K > 0 ? s0 : s1, 0, m0, n0, M, N, tid, ra, rb);
    store_stage<T>(nst0 > 0 ? s0 : s1, tid, ra, rb, As[0], Bs[0]);
    __syncthreads();
    for (int st = 0; st < total; ++st) {
      const int nx = st + 1;
      const bool more = nx < total;
      const bool nx_first = nx < nst0;
      if (more) load_stage<T>(nx_first ? s0 : s1, (nx_first ? nx : nx - nst0) * KBK, m0, n0, M, N, tid, ra, rb);
      const int buf = st & 1;
#pragma unroll
      for (int kq = 0; kq < KBK / 4; ++kq) {
        const int kr = kq * 4 + (lane >> 4);
        T a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[buf][kr][wm + 16 * i + arow];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[buf][kr][wn + 16 * j + (lane & 15)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = Mfma<T>::mma(a[i], b[j], acc[i][j]);
      }
      if (more) store_stage<T>(nx_first ? s0 : s1, tid, ra, rb, As[buf ^ 1], Bs[buf ^ 1]);
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+v, column lane%16 of each 16x16 tile
  T *C = static_cast<T *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;
  const bool fin = t.final_ != 0;
  const bool rd = fin && beta != T(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn + 16 * j + (lane & 15);
    if (n >= N) continue;
    const int64_t col = t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n];
    T *cp = C + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mb = m0 + wm + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mb + v;
        if (m < M) {
          T x = acc[i][j][v];
          if (fin) {
            x = alpha * x;
            if (rd) x += beta * cp[m];
          }
          cp[m] = x;
        }
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(NTHR) void grouped_gemm_kernel(const DevTask *__restrict__ tasks,
                                                            const DevTile *__restrict__ tiles,
                                                            const int64_t *__restrict__ coltab,
                                                            Bases bases, T alpha, T beta) {
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
__global__ __launch_bounds__(NTHR) void single_gemm_kernel(DevTask t, Bases bases, T alpha, T beta,
                                                           int mt, int nt, int per) {
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

}  // namespace

int launch_grouped(tlr_dtype dt, const DevTask *tasks, const DevTile *tiles, int64_t n_tiles,
                   const int64_t *coltab, const Bases &bases, double alpha, double beta, void *stream) {
  if (n_tiles <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)n_tiles), block(NTHR);
  if (dt == TLR_F64)
    hipLaunchKernelGGL(grouped_gemm_kernel<double>, grid, block, 0, s, tasks, tiles, coltab, bases, alpha, beta);
  else
    hipLaunchKernelGGL(grouped_gemm_kernel<float>, grid, block, 0, s, tasks, tiles, coltab, bases,
                       (float)alpha, (float)beta);
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
