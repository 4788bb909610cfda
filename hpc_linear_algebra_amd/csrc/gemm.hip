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
// Work split: the 128 x 128 block is shared by 4 or 8 wave64s (64 x 64 or
// 64 x 32 per wave, MFMA tiles of 16 x 16: v_mfma_f64_16x16x4_f64 /
// v_mfma_f32_16x16x4_f32).  K advances in stages of BK = 16, staged through LDS
// and double-buffered: the global loads of stage s+1 are in flight while the
// MFMAs of stage s run.  Registers are held so that two workgroups share a CU:
// while one waits on memory (its first stage, its C update) the other keeps
// the matrix cores busy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tlr_plan.h"

namespace tlr {

namespace {

// LDS rows hold 145 elements: an odd stride sends the 16 k-rows that one
// K-contiguous operand store touches to 16 different banks, and a 16-element
// fragment read still covers each bank once.
constexpr int KBM = 128, KBN = 128, KBK = 16, KPAD = 17;
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

// Wave layout of a 128 x 128 workgroup block: WM x WN per wave (MI x NJ MFMA
// tiles of 16 x 16), NT threads.  64 x 64 waves (4 per workgroup) hold 128
// accumulator registers; 64 x 32 waves (8 per workgroup) hold 64, which lets
// two workgroups keep four waves on every SIMD.
template <int WM_, int WN_> struct Layout {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int WAVES_M = KBM / WM, WAVES_N = KBN / WN;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int MI = WM / 16, NJ = WN / 16;
  static constexpr int EPT = KBM * KBK / NT;     // elements per thread per operand per stage
  static constexpr int WPE = NW / 2;             // waves per SIMD with two workgroups per CU
};

// Which EPT elements of a 128 x 16 (A) or 16 x 128 (B) stage one thread moves.
// When the 128-long index x (m for A, n for B) is the contiguous one, lanes
// walk x and each thread takes k = k0, k0+NT/128, ...; otherwise lanes walk k
// and each thread takes x = x0, x0+NT/16, ....  Element p sits at intra-tile
// offset lin + p*step of the operand and at LDS index lds + p*lds_step.
struct ThreadMap {
  int32_t lin, step;
  int32_t x, dx, k, dk;
  int32_t lds, lds_step;
};

template <int NT>
__device__ __forceinline__ ThreadMap thread_map(bool x_contig, int32_t ld, int tid, int lds_row) {
  ThreadMap t;
  if (x_contig) {
    const int x = tid & 127, k = tid >> 7;
    constexpr int dk = NT / 128;
    t.lin = x + k * ld; t.step = dk * ld;
    t.x = x; t.dx = 0; t.k = k; t.dk = dk;
    t.lds = k * lds_row + x; t.lds_step = dk * lds_row;
  } else {
    const int k = tid & 15, x = tid >> 4;
    constexpr int dx = NT / 16;
    t.lin = k + x * ld; t.step = dx * ld;
    t.x = x; t.dx = dx; t.k = k; t.dk = 0;
    t.lds = k * lds_row + x; t.lds_step = dx;
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

template <typename T, int NT>
__device__ __forceinline__ Seg<T> make_seg(const DevSeg &g, const Bases &bases, int tid) {
  Seg<T> s;
  s.a = static_cast<const T *>(bases.p[g.a.base]) + g.a.off;
  s.b = static_cast<const T *>(bases.p[g.b.base]) + g.b.off;
  s.lda = g.a.ld;
  s.ldb = g.b.ld;
  s.K = g.K;
  s.a_xc = g.a.trans == 0;   // A(m,k) = A[m + k*lda]
  s.b_xc = g.b.trans == 1;   // B(k,n) = B[n + k*ldb]
  s.ma = thread_map<NT>(s.a_xc, s.lda, tid, LDS_A);
  s.mb = thread_map<NT>(s.b_xc, s.ldb, tid, LDS_B);
  return s;
}

// Operand loads are raw buffer loads from a resource whose base is the tile
// origin: an element outside the operand gets the offset 2^31, which lies past
// the resource's 2^31 - 1 byte range, and the hardware returns zero for it
// without touching memory.  Valid elements are at byte offsets below 2^31
// (leading dimensions are below 2^21), so no select or branch follows the loads
// and all eight of a thread's loads can be in flight together.
template <typename T> struct BufLoad;
template <> struct BufLoad<double> {
  static __device__ __forceinline__ double ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
};
template <> struct BufLoad<float> {
  static __device__ __forceinline__ float ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
};

constexpr uint32_t OOB_OFFSET = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;   // raw (untyped) buffer access on CDNA

template <typename T, int EPT>
__device__ __forceinline__ void load_op(const T *base, int64_t x0, int64_t k0, int32_t ld, bool xc, int xrem,
                                        int krem, const ThreadMap &m, T (&r)[EPT]) {
  const T *p0 = xc ? base + x0 + k0 * ld : base + k0 + x0 * ld;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(p0), (short)0, 0x7fffffff, BUF_WORD3);
#pragma unroll
  for (int p = 0; p < EPT; ++p) {
    const int x = m.x + p * m.dx, k = m.k + p * m.dk;
    const bool ok = x < xrem && k < krem;
    const uint32_t off = ok ? (uint32_t)(m.lin + p * m.step) * (uint32_t)sizeof(T) : OOB_OFFSET;
    r[p] = BufLoad<T>::ld(rs, off);
  }
}

template <typename T, int EPT>
__device__ __forceinline__ void load_stage(const Seg<T> &s, int k0, int m0, int n0, int M, int N,
                                           T (&ra)[EPT], T (&rb)[EPT]) {
  const int krem = s.K - k0;
  load_op<T, EPT>(s.a, m0, k0, s.lda, s.a_xc, M - m0, krem, s.ma, ra);
  load_op<T, EPT>(s.b, n0, k0, s.ldb, s.b_xc, N - n0, krem, s.mb, rb);
}

template <typename T, int EPT>
__device__ __forceinline__ void store_stage(const Seg<T> &s, const T (&ra)[EPT], const T (&rb)[EPT], T *As, T *Bs) {
#pragma unroll
  for (int p = 0; p < EPT; ++p) As[s.ma.lds + p * s.ma.lds_step] = ra[p];
#pragma unroll
  for (int p = 0; p < EPT; ++p) Bs[s.mb.lds + p * s.mb.lds_step] = rb[p];
}

template <typename T, typename L>
__device__ __forceinline__ void gemm_block(const DevTask &t, int m0, int n0, const int64_t *coltab,
                                           const Bases &bases, T alpha, T beta, T cscale) {
  typedef typename Mfma<T>::v4 v4;
  constexpr int MI = L::MI, NJ = L::NJ, EPT = L::EPT;
  __shared__ T As[2][KBK * LDS_A];
  __shared__ T Bs[2][KBK * LDS_B];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave % L::WAVES_M) * L::WM, wn = (wave / L::WAVES_M) * L::WN;
  const int arow = Mfma<T>::arow(lane & 15);
  const int M = t.M, N = t.N;

  // C <- alpha*(acc + (beta/alpha)*C): when the host found beta/alpha finite the
  // old C is read into the accumulators before the K loop (its latency hides
  // behind the first loads) and the epilogue only stores.
  T *C = static_cast<T *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;
  const bool fin = t.final_ != 0;
  const bool vec = (t.flags & TASK_VEC) && (reinterpret_cast<uintptr_t>(C) % (4 * sizeof(T)) == 0);
  const bool preload = fin && cscale != T(0);
  const bool rd = fin && beta != T(0) && !preload;
  v4 acc[MI][NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + (lane & 15);
    const int64_t col = (!preload || n >= N) ? 0 : (t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n]);
    const T *cp = C + col;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      acc[i][j] = v4{0, 0, 0, 0};
      if (!preload || n >= N) continue;
      const int mb = m0 + wm + 16 * i + 4 * (lane >> 4);
      if (vec && mb + 3 < M) {
        acc[i][j] = cscale * *reinterpret_cast<const v4 *>(cp + mb);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (mb + v < M) acc[i][j][v] = cscale * cp[mb + v];
      }
    }
  }

  const int nseg = t.nseg;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {   // constant segment index: no dynamic indexing into the task
    if (sg >= nseg) break;
    const Seg<T> s = make_seg<T, L::NT>(t.seg[sg], bases, tid);
    const int nst = (s.K + KBK - 1) / KBK;
    T ra[EPT], rb[EPT];
    load_stage<T, EPT>(s, 0, m0, n0, M, N, ra, rb);
    __syncthreads();   // the previous segment's last reads of buffer 0 are done
    store_stage<T, EPT>(s, ra, rb, As[0], Bs[0]);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const bool more = st + 1 < nst;
      if (more) load_stage<T, EPT>(s, (st + 1) * KBK, m0, n0, M, N, ra, rb);
      const T *Ab = As[st & 1];
      const T *Bb = Bs[st & 1];
#pragma unroll
      for (int kq = 0; kq < KBK / 4; ++kq) {
        const int kr = kq * 4 + (lane >> 4);
        T a[MI], b[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i) a[i] = Ab[kr * LDS_A + wm + 16 * i + arow];
#pragma unroll
        for (int j = 0; j < NJ; ++j) b[j] = Bb[kr * LDS_B + wn + 16 * j + (lane & 15)];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = Mfma<T>::mma(a[i], b[j], acc[i][j]);
      }
      if (more) store_stage<T, EPT>(s, ra, rb, As[(st + 1) & 1], Bs[(st + 1) & 1]);
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+v (v = 0..3), column lane%16 of each
  // 16x16 tile; when the column start is 4-element aligned those four rows go
  // out as one vector access.
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + (lane & 15);
    if (n >= N) continue;
    const int64_t col = t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n];
    T *cp = C + col;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
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

template <typename T, int STAGE, typename L>
__global__ __launch_bounds__(L::NT) __attribute__((amdgpu_waves_per_eu(L::WPE)))
void grouped_gemm_kernel(const DevTask *__restrict__ tasks, const DevTile *__restrict__ tiles,
                         const int64_t *__restrict__ coltab, Bases bases, T alpha, T beta, T cscale) {
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask t = tasks[e.task];
  const bool fin = t.final_ != 0;
  gemm_block<T, L>(t, e.m0, e.n0, coltab, bases, fin ? alpha : T(1), fin ? beta : T(0), fin ? cscale : T(0));
}

// Single task given by value; blockIdx.x walks the output blocks so that each
// XCD (workgroups are dealt to the 8 XCDs round-robin) takes a contiguous run
// of block indices, ordered in bands of 8 block rows for L2 reuse.
template <typename T, typename L>
__global__ __launch_bounds__(L::NT) __attribute__((amdgpu_waves_per_eu(L::WPE)))
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
  gemm_block<T, L>(t, mtile * KBM, ntile * KBN, nullptr, bases, alpha, beta, cscale);
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
// epilogue reads C).
template <typename T>
T preload_scale(double alpha, double beta) {
  if (beta == 0.0 || alpha == 0.0) return T(0);
  const double r = beta / alpha;
  const double lim = sizeof(T) == 8 ? 1e300 : 1e30;
  return (r == r && r < lim && r > -lim) ? T(r) : T(0);
}

// 64 x 32 waves (8 per workgroup, four waves per SIMD with two workgroups per
// CU) measured faster than 64 x 64 waves at every K on this chip: more waves
// cover the barrier and memory phases of a workgroup.
using WaveLayout = Layout<64, 32>;

template <typename T, typename L>
void launch_grouped_l(int stage, unsigned n, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                      const int64_t *coltab, const Bases &bases, T a, T b, T c) {
  dim3 grid(n), block(L::NT);
  if (stage == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 1, L>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else if (stage == 2)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 2, L>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 3, L>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
}

template <typename T>
void launch_grouped_t(int stage, unsigned n, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                      const int64_t *coltab, const Bases &bases, double alpha, double beta) {
  const T a = (T)alpha, b = (T)beta, c = preload_scale<T>(alpha, beta);
  launch_grouped_l<T, WaveLayout>(stage, n, s, tasks, tiles, coltab, bases, a, b, c);
}

template <typename T>
void launch_single_t(unsigned n, hipStream_t s, const DevTask &task, const Bases &bases, double alpha,
                     double beta, int mt, int nt, int per) {
  const T a = (T)alpha, b = (T)beta, c = preload_scale<T>(alpha, beta);
  hipLaunchKernelGGL((single_gemm_kernel<T, WaveLayout>), dim3(n), dim3(WaveLayout::NT), 0, s, task, bases, a, b,
                     c, mt, nt, per);
}

}  // namespace

int launch_grouped(tlr_dtype dt, int stage, const DevTask *tasks, const DevTile *tiles, int64_t n_tiles,
                   const int64_t *coltab, const Bases &bases, double alpha, double beta, void *stream) {
  if (n_tiles <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F64)
    launch_grouped_t<double>(stage, (unsigned)n_tiles, s, tasks, tiles, coltab, bases, alpha, beta);
  else
    launch_grouped_t<float>(stage, (unsigned)n_tiles, s, tasks, tiles, coltab, bases, alpha, beta);
  return (int)hipGetLastError();
}

int launch_single(tlr_dtype dt, const DevTask &task, const Bases &bases, double alpha, double beta,
                  void *stream) {
  const int mt = (task.M + KBM - 1) / KBM, nt = (task.N + KBN - 1) / KBN;
  if (mt == 0 || nt == 0) return 0;
  const int64_t n = (int64_t)mt * nt;
  const int per = (int)((n + 7) / 8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F64)
    launch_single_t<double>((unsigned)(per * 8), s, task, bases, alpha, beta, mt, nt, per);
  else
    launch_single_t<float>((unsigned)(per * 8), s, task, bases, alpha, beta, mt, nt, per);
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
