// Dense <-> TLR conversions on the GPU: the pieces of a product whose output
// C is itself TLR ("TLR Matrix Multiplication", "Introduction: TLR GEMM": A, B
// and C may each be dense or TLR; the TLR-output cases extend the
// dense-output product).
//
//   tlr_expand    C <- alpha X + beta C for a stored TLR operand X (every tile
//                 U_ij V_ij^T, dense diagonal tiles), C dense.
//   tlr_compress  a dense matrix to TLR: dense diagonal tiles, and every other
//                 tile replaced by its truncated SVD of the smallest rank whose
//                 discarded part meets a relative Frobenius tolerance.
//
// Compression of one tile X (s_i x s_j), with s = max_rank + 8 samples:
//   Y  = X Omega          (s_i x s)  range sketch, Omega given by the caller
//   Y  = Q R              Householder QR, Q kept (s_i x s)
//   Bt = X^T Q            (s_j x s)  so that X ~ Q Bt^T = Q Q^T X
//   Bt = Q2 R2            Householder QR, Q2 (s_j x s) and R2 (s x s) kept
//   M  = R2^T             X ~ Q M Q2^T
//   M J = W               one-sided (Hestenes) Jacobi: J orthogonal, the
//                         columns of W orthogonal with norms sigma_k
//   X ~ (Q W) (Q2 J)^T    U = Q W (columns of norm sigma), V = Q2 J
// The energy Q misses is ||X||_F^2 - sum sigma_k^2; the kept rank r is the
// smallest for which that energy plus the discarded sigma_k^2 stays within
// (tol ||X||_F)^2.  The products run on the tile-batched MFMA GEMM; QR,
// Jacobi, the rank scan and the packing are kernels of this file, one
// workgroup per tile.  Ranks and factor offsets stay on the device: nothing
// here synchronises with the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "tlr_plan.h"

namespace tlr {

namespace {

constexpr int CT = 256;          // threads of the per-tile kernels (four wave64s)
constexpr int OVERSAMPLE = 8;    // samples beyond max_rank
constexpr int S_MAX = 64;        // largest sample count (max_rank <= 56)

__device__ __forceinline__ int tile_rows(int64_t n, int64_t b, int i) { return (int)min<int64_t>(b, n - (int64_t)i * b); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the workgroup of NTH threads (every thread gets it).  red holds
// NTH/64 slots.
template <typename T, int NTH = CT>
__device__ __forceinline__ T block_sum(T v, T *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T s = 0;
#pragma unroll
  for (int k = 0; k < NTH / 64; ++k) s += red[k];
  return s;
}

// ||X_t||_F^2 of every tile.
template <typename T>
__global__ __launch_bounds__(CT) void tile_norms_kernel(const T *X, int64_t ldx, int qr, int qc, int64_t rows,
                                                       int64_t cols, int64_t b, T *norms2) {
  __shared__ T red[CT / 64];
  const int t = blockIdx.x;
  const int i = t % qr, j = t / qr;
  const int si = tile_rows(rows, b, i), sj = tile_rows(cols, b, j);
  const T *x = X + (int64_t)i * b + (int64_t)j * b * ldx;
  // eight columns per step with their own partial sums: eight loads in
  // flight per thread instead of one serial chain
  constexpr int CU = 8;
  T part[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) part[u] = 0;
  for (int r = threadIdx.x; r < si; r += CT) {
    int c = 0;
    for (; c + CU <= sj; c += CU) {
      T v[CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) v[u] = x[r + (int64_t)(c + u) * ldx];
#pragma unroll
      for (int u = 0; u < CU; ++u) part[u] += v[u] * v[u];
    }
    for (; c < sj; ++c) {
      const T v = x[r + (int64_t)c * ldx];
      part[0] += v * v;
    }
  }
  T acc = 0;
#pragma unroll
  for (int u = 0; u < CU; ++u) acc += part[u];
  acc = block_sum(acc, red);
  if (threadIdx.x == 0) norms2[t] = acc;
}

// Householder QR of one m x n panel a (column-major, leading dim lda; in LDS
// or global memory), n <= S_MAX, by a workgroup of NTH threads, with at most
// kcap reflectors.  The panel is overwritten by the explicit Q (m x n,
// orthonormal columns; columns past min(m, n, kcap) zero); with rr != nullptr the n x n upper factor is written to rr
// (column-major, zero below the diagonal).  Reflector k: v = x - alpha e_k with
// alpha = -sign(x_k) ||x||, H = I - beta v v^T, beta = 2 / (v^T v); v stays in
// column k (rows >= k) until Q is formed.
template <typename T, int NTH>
__device__ __forceinline__ void qr_panel(T *a, int lda, T *rr, int m, int n, int kcap, T *red, T *beta_s) {
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kmax = min(min(m, n), kcap);
  if (rr)
    for (int e = tid; e < n * n; e += NTH) rr[e] = 0;
  for (int k = 0; k < kmax; ++k) {
    T tail = 0;
    for (int r = k + 1 + tid; r < m; r += NTH) {
      const T v = a[r + (int64_t)k * lda];
      tail += v * v;
    }
    tail = block_sum<T, NTH>(tail, red);
    const T x0 = a[k + (int64_t)k * lda];
    const T nrm = sqrt(tail + x0 * x0);
    const T alpha = x0 >= T(0) ? -nrm : nrm;
    const T v0 = x0 - alpha;
    const T vtv = tail + v0 * v0;
    const T beta = vtv > T(0) ? T(2) / vtv : T(0);
    __syncthreads();   // every thread has read x0 before it is replaced
    if (tid == 0) {
      a[k + (int64_t)k * lda] = v0;
      beta_s[k] = beta;
      if (rr) rr[k + (int64_t)k * n] = alpha;
    }
    __syncthreads();
    // trailing columns: A[k:m, c] -= beta (v^T A[k:m, c]) v, one wave per column
    for (int c = k + 1 + wave; c < n; c += NW) {
      T sacc = 0;
      for (int r = k + lane; r < m; r += 64) sacc += a[r + (int64_t)k * lda] * a[r + (int64_t)c * lda];
      sacc = wave_sum(sacc);
      const T f = beta * sacc;
      for (int r = k + lane; r < m; r += 64) a[r + (int64_t)c * lda] -= f * a[r + (int64_t)k * lda];
      if (rr && lane == 0) rr[k + (int64_t)c * n] = a[k + (int64_t)c * lda];
    }
    __syncthreads();
  }
  // Q = H_0 ... H_{kmax-1} applied to the first n columns of the identity,
  // formed backwards in place; columns past kmax are zero
  for (int c = kmax; c < n; ++c)
    for (int r = tid; r < m; r += NTH) a[r + (int64_t)c * lda] = 0;
  __syncthreads();
  for (int k = kmax - 1; k >= 0; --k) {
    const T beta = beta_s[k];
    for (int c = k + 1 + wave; c < n; c += NW) {
      // rows < k+1 of column c are zero here, so the sum starts at k + 1
      T sacc = 0;
      for (int r = k + 1 + lane; r < m; r += 64) sacc += a[r + (int64_t)k * lda] * a[r + (int64_t)c * lda];
      sacc = wave_sum(sacc);
      const T f = beta * sacc;
      // row k of column c becomes -f v0
      if (lane == 0) a[k + (int64_t)c * lda] = -f * a[k + (int64_t)k * lda];
      for (int r = k + 1 + lane; r < m; r += 64) a[r + (int64_t)c * lda] -= f * a[r + (int64_t)k * lda];
    }
    __syncthreads();
    const T v0 = a[k + (int64_t)k * lda];
    __syncthreads();   // v0 read by every thread before column k is rewritten
    for (int r = tid; r < m; r += NTH) {
      const T vr = a[r + (int64_t)k * lda];
      a[r + (int64_t)k * lda] = r < k ? T(0) : (r == k ? T(1) - beta * v0 * v0 : -beta * v0 * vr);
    }
    __syncthreads();
  }
}

constexpr int QR_ROWS = 256;   // rows of a register-resident panel (b <= 256)

// How a QR launch treats the per-tile column count kq (the columns of the
// sketch basis Q that the later steps use):
//   KQ_SET  the QR of the sketches: stop early where the sketch shows the
//           rest of the tile to be negligible (qr_reg_kernel), write kq[t];
//   KQ_CAP  the QR of the projections: at most kq[t] reflectors.
enum KqMode : int { KQ_SET = 1, KQ_CAP = 2 };

// QR of every tile's m x n panel (tile t at A + t * stride, leading dim lda),
// m = s_i (m_sel 0) or s_j (m_sel 1); R (optional) at R + t * n * n,
// factorised in place in global memory by CT threads (tiles of more than
// QR_ROWS rows; smaller ones take qr_reg_kernel below).
template <typename T>
__global__ __launch_bounds__(CT) void qr_tiles_kernel(T *A, int lda, int64_t stride, T *R, int qr, int qc,
                                                       int64_t rows, int64_t cols, int64_t b, int m_sel, int n,
                                                       int skip_diag, int32_t *kq, int kq_mode) {
  __shared__ T red[CT / 64];
  __shared__ T beta_s[S_MAX];
  const int t = blockIdx.x;
  const int i = t % qr, j = t / qr;
  if (skip_diag && i == j) return;
  const int m = m_sel == 0 ? tile_rows(rows, b, i) : tile_rows(cols, b, j);
  T *a = A + (int64_t)t * stride;
  T *rr = R ? R + (int64_t)t * n * n : nullptr;
  const int kcap = kq_mode == KQ_CAP ? kq[t] : n;
  qr_panel<T, CT>(a, lda, rr, m, n, kcap, red, beta_s);
  if (kq_mode == KQ_SET && threadIdx.x == 0) kq[t] = min(m, n);
}

// The same QR for panels of at most QR_ROWS rows, held in registers.  Thread
// (c, p) of QRR_THREADS (8 consecutive lanes per column) holds column c of the
// panel at rows p, p + 8, ..., p + 248 (QRR_REGS registers, zero past m) for
// the whole factorisation and for the forming of Q.  Reflector k:
//   * the 8 threads of column k form the tail norm (an 8-lane sum), alpha,
//     beta and v, write v (zero above row k) into an LDS buffer and beta into
//     beta_s, and keep v below their R part;
//   * one barrier;
//   * the threads of every column c > k read v at their rows, form their part
//     of w_c = v^T A[:, c], sum the 8 parts (part_sum8) and update their
//     registers: A[:, c] -= beta v w_c.
// Rows above k of a column c > k hold finished entries of R; v is zero there,
// so they drop out without a mask.  The v buffers alternate, so the readers of
// one reflector and the writers of the next never meet: one barrier per
// reflector and 2 KB of LDS traffic, where a panel kept in LDS moves through
// it at every reflector (its update was bound by LDS bandwidth).  Row k sits
// in register k / 8 of lane k % 8: the reflectors go in blocks of 8 with the
// loop over blocks unrolled, so every register index is static.  Q is formed
// backwards the same way: the threads of column k broadcast v_k, then hold
// column k of Q (H_k e_k); the columns c > k take H_k.
//
// With KQ_SET (the QR of the sketches Y = X Omega, Omega Gaussian) the
// factorisation stops after a multiple of 4 reflectors once the rest of the
// sketch is negligible: after k reflectors the rows >= k of the columns
// c >= k hold the parts of y_c = X omega_c outside the span P_k of the first
// k columns, and P_k depends on omega_0 .. omega_{k-1} only, so their energy
// E is a sum of n - k independent samples of ||(I - P_k) X omega||^2, whose
// mean is ||(I - P_k) X||_F^2 (the posterior error estimate of the
// randomized range finder).  The QR stops at k when E <= stop (n - k)
// ||X||_F^2 with at least OVERSAMPLE samples left; the energy it leaves out
// of the basis then stays below 1e3 stop ||X||_F^2 unless a chi-square
// variable of n - k >= 8 degrees of freedom falls under 1e-3 of its mean
// (probability below 1e-11).  Q keeps k columns (the rest zero) and kq[t] = k
// caps the QR of the projections and the Jacobi SVD that follow.
constexpr int QRR_PARTS = 8;                      // threads per column
constexpr int QRR_REGS = QR_ROWS / QRR_PARTS;     // rows per thread
constexpr int QRR_THREADS = QRR_PARTS * S_MAX;    // 512
constexpr int QRR_BLOCKS = S_MAX / QRR_PARTS;     // blocks of 8 reflectors

// Sum over each group of 8 consecutive lanes, every lane getting it, with
// DPP lane moves (VALU, no LDS round trip): partner i ^ 1 and i ^ 2 by quad
// permutations, then the other half of the 8 by the half-row mirror (lane i
// of a group reads lane 7 - i, which after two steps holds the other quad's
// sum).  Each step adds a pair in either order, so all lanes agree exactly.
template <int CTRL>
__device__ __forceinline__ double dpp_move(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// x from lane `lane` of the wave (a wave-uniform lane index: v_readlane)
__device__ __forceinline__ double lane_value(double x, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;  // row_half_mirror
template <typename T>
__device__ __forceinline__ T part_sum8(T x) {
  x += dpp_move<DPP_QUAD_XOR1>(x);
  x += dpp_move<DPP_QUAD_XOR2>(x);
  x += dpp_move<DPP_HALF_MIRROR>(x);
  return x;
}

template <typename T>
__global__ __launch_bounds__(QRR_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void qr_reg_kernel(T *A, int lda, int64_t stride, T *R, int qr, int qc,
                                                            int64_t rows, int64_t cols, int64_t b, int m_sel, int n,
                                                            int skip_diag, int32_t *kq, int kq_mode,
                                                            const T *norms2, T stop) {
  __shared__ T vbuf[2][QR_ROWS];
  __shared__ T beta_s[S_MAX];
  __shared__ T ctail[S_MAX];
  const int t = blockIdx.x;
  const int i = t % qr, j = t / qr;
  if (skip_diag && i == j) return;
  const int m = m_sel == 0 ? tile_rows(rows, b, i) : tile_rows(cols, b, j);
  T *a = A + (int64_t)t * stride;
  T *rr = R ? R + (int64_t)t * n * n : nullptr;
  const int tid = threadIdx.x, c = tid / QRR_PARTS, p = tid % QRR_PARTS;
  int kmax = min(m, n);   // the same in every thread
  // columns that can be nonzero: with KQ_CAP those past kq[t] are zero (the
  // sketch basis has kq[t] columns) and stay zero under every reflector
  const int ncol = kq_mode == KQ_CAP ? min(n, kq[t]) : n;
  kmax = min(kmax, ncol);
  T y[QRR_REGS];
#pragma unroll
  for (int q = 0; q < QRR_REGS; ++q) {
    const int r = QRR_PARTS * q + p;
    y[q] = (c < n && r < m) ? a[r + (int64_t)c * lda] : T(0);
  }
  if (rr)
    for (int e = tid; e < n * n; e += QRR_THREADS) rr[e] = 0;
  __syncthreads();

  // v of reflector k = 8K + kk into vb (rows >= 8K; zero above row k), from
  // the registers of column k, whose row k holds v0
  auto put_v = [&](T *vb, auto Kc, int kk, T v0) {
    constexpr int K = decltype(Kc)::value;
#pragma unroll
    for (int q = K; q < QRR_REGS; ++q)
      vb[QRR_PARTS * q + p] = q > K ? y[q] : (p > kk ? y[K] : (p == kk ? v0 : T(0)));
  };
  // A[:, c] -= beta v (v^T A[:, c]) for this thread's column
  auto reflect = [&](const T *vb, auto Kc, T beta) {
    constexpr int K = decltype(Kc)::value;
    // four partial sums: chains of at most 8 dependent FMAs
    T w4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int q = K; q < QRR_REGS; ++q) w4[(q - K) & 3] += vb[QRR_PARTS * q + p] * y[q];
    const T bw = beta * part_sum8((w4[0] + w4[1]) + (w4[2] + w4[3]));
    // v is read again rather than held: 32 more registers would leave one
    // workgroup per CU instead of two
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = K; q < QRR_REGS; ++q) y[q] -= vb[QRR_PARTS * q + p] * bw;
  };

  // factorisation
  auto forward = [&](auto Kc) {
    constexpr int K = decltype(Kc)::value;
    for (int kk = 0; kk < QRR_PARTS; ++kk) {
      const int k = QRR_PARTS * K + kk;
      if (k >= kmax) break;
      T *vb = vbuf[k & 1];
      if (c == k) {
        T t4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = K; q < QRR_REGS; ++q)
          if (q > K || p > kk) t4[(q - K) & 3] += y[q] * y[q];
        const T tail = part_sum8((t4[0] + t4[1]) + (t4[2] + t4[3]));
        // row k: register K of lane kk of column k's lanes (wave k / 8)
        const T x0 = lane_value(y[K], QRR_PARTS * (k % (64 / QRR_PARTS)) + kk);
        const T nrm = sqrt(tail + x0 * x0);
        const T alpha = x0 >= T(0) ? -nrm : nrm;
        const T v0 = x0 - alpha;
        const T vtv = tail + v0 * v0;
        const T beta = vtv > T(0) ? T(2) / vtv : T(0);
        put_v(vb, Kc, kk, v0);
        if (p == kk) y[K] = v0;
        if (p == 0) {
          beta_s[k] = beta;
          if (rr) rr[k + k * n] = alpha;
        }
      }
      __syncthreads();
      if (c > k && c < ncol) reflect(vb, Kc, beta_s[k]);
      // the early stop after every fourth reflector: E from the rows >= KN
      // of the columns >= KN, summed in column order (the same value, so the
      // same decision, in every thread)
      const int KN = k + 1;
      if (kq_mode == KQ_SET && (kk & 3) == 3 && KN < kmax && KN + OVERSAMPLE <= n) {
        T t4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = K; q < QRR_REGS; ++q)
          if (q > K || p > kk) t4[(q - K) & 3] += y[q] * y[q];
        const T tl = part_sum8((t4[0] + t4[1]) + (t4[2] + t4[3]));
        if (p == 0 && c >= KN && c < n) ctail[c] = tl;
        __syncthreads();   // the next write of ctail is four reflectors later
        T e = 0;
        for (int x = KN; x < n; ++x) e += ctail[x];
        if (e <= stop * T(n - KN) * norms2[t]) kmax = KN;
      }
    }
  };
  forward(std::integral_constant<int, 0>());
  forward(std::integral_constant<int, 1>());
  forward(std::integral_constant<int, 2>());
  forward(std::integral_constant<int, 3>());
  forward(std::integral_constant<int, 4>());
  forward(std::integral_constant<int, 5>());
  forward(std::integral_constant<int, 6>());
  forward(std::integral_constant<int, 7>());
  static_assert(QRR_BLOCKS == 8, "one forward/backward call per block of 8 reflectors");
  if (kq_mode == KQ_SET && tid == 0) kq[t] = kmax;

  // R above the diagonal: rows r < c of column c are final
  if (rr && c < n) {
#pragma unroll
    for (int q = 0; q < QRR_REGS; ++q) {
      const int r = QRR_PARTS * q + p;
      if (r < c && r < kmax) rr[r + c * n] = y[q];
    }
  }
  // columns past the last reflector are zero in Q
  if (c >= kmax) {
#pragma unroll
    for (int q = 0; q < QRR_REGS; ++q) y[q] = 0;
  }
  __syncthreads();   // the last reflector's readers are done with its v buffer

  // Q = H_0 ... H_{kmax-1} [I; 0], formed backwards
  auto backward = [&](auto Kc) {
    constexpr int K = decltype(Kc)::value;
    for (int kk = QRR_PARTS - 1; kk >= 0; --kk) {
      const int k = QRR_PARTS * K + kk;
      if (k >= kmax) continue;
      T *vb = vbuf[k & 1];
      const T beta = beta_s[k];
      if (c == k) {
        const T v0 = lane_value(y[K], QRR_PARTS * (k % (64 / QRR_PARTS)) + kk);
        put_v(vb, Kc, kk, v0);
        // column k of Q: H_k e_k
#pragma unroll
        for (int q = 0; q < QRR_REGS; ++q) {
          const int r = QRR_PARTS * q + p;
          y[q] = q < K ? T(0) : (r == k ? T(1) - beta * v0 * v0 : (r > k ? -beta * v0 * y[q] : T(0)));
        }
      }
      __syncthreads();
      if (c > k && c < kmax) reflect(vb, Kc, beta);   // the columns past kmax are zero
    }
  };
  backward(std::integral_constant<int, 7>());
  backward(std::integral_constant<int, 6>());
  backward(std::integral_constant<int, 5>());
  backward(std::integral_constant<int, 4>());
  backward(std::integral_constant<int, 3>());
  backward(std::integral_constant<int, 2>());
  backward(std::integral_constant<int, 1>());
  backward(std::integral_constant<int, 0>());

  if (c < n) {
#pragma unroll
    for (int q = 0; q < QRR_REGS; ++q) {
      const int r = QRR_PARTS * q + p;
      if (r < m) a[r + (int64_t)c * lda] = y[q];
    }
  }
}

// Threads per column pair: 8 consecutive lanes of one wave take rows part,
// part + 8, ... of a pair and combine their partial sums with lane shuffles.
constexpr int JPARTS = 8;
// M and J live in dynamic LDS sized to the tile: np columns of 8 RPL rows
// (RPL = jacobi_rpl(np) rows per lane of a pair, the rows past n zero) at
// stride jacobi_ld(RPL) = 8 RPL + 2 (2 x 56 x 58 doubles at the sketch width
// 56, 52 KB: three workgroups per CU, where arrays sized for S_MAX took 74 KB
// and allowed two).  An even stride that is not a multiple of 32 doubles
// starts the eight columns a wave reads at once on different banks.
__host__ __device__ constexpr int jacobi_rpl(int np) { return (np + JPARTS - 1) / JPARTS; }
__host__ __device__ constexpr int jacobi_ld(int rpl) { return JPARTS * rpl + 2; }
__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }

// One-sided Jacobi SVD of M = R2^T (n x n, R2 of every tile at R + t n n;
// its rows and columns from kq[t] on are zero, so only the first kq[t]
// columns take part in the rotations), then the rank at the tolerance.  Writes W = M J (n x n, column k of norm
// sigma_k) to Wout + t n n, J to Jout + t n n, the columns in decreasing
// order of sigma to perm + t n, the rank to ranks[t] (0 for a skipped
// diagonal tile) and flags[t] = 1 when the tolerance was not met within
// max_rank columns (the rank is then max_rank); jstat[2t], jstat[2t + 1] =
// the pairs visited (sweeps x pairs x rounds: the 2 x 2 Gram blocks formed)
// and the rotations applied (the measure of its work).
// RPL = jacobi_rpl(np) is a compile-time count, so the row loops of a round
// run without guards: the kernel is bound by VALU issue, not by LDS.
template <typename T, int RPL>
__global__ __launch_bounds__(CT) void jacobi_rank_kernel(const T *R, T *Wout, T *Jout, int32_t *perm,
                                                        int32_t *ranks, int32_t *flags, int32_t *jstat,
                                                        const T *norms2, const int32_t *kq, int qr, int qc, int n,
                                                        int max_rank, T tol, T conv, int skip_diag) {
  extern __shared__ __attribute__((aligned(16))) unsigned char jacobi_lds[];
  __shared__ T sig2[S_MAX];
  __shared__ int order[S_MAX];
  __shared__ T offw[2][32];           // [sweep % 2][pair]: the pair slot's largest cos^2 in the sweep
  const int t = blockIdx.x;
  const int i = t % qr, j = t / qr;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (skip_diag && i == j) {
    if (tid == 0) {
      ranks[t] = 0;
      flags[t] = 0;
      jstat[2 * t] = 0;
      jstat[2 * t + 1] = 0;
    }
    return;
  }
  __shared__ int nrot;
  if (tid == 0) nrot = 0;
  const int nall = (n + 1) & ~1;        // columns held in LDS (a zero column when n is odd)
  const int np = (min(n, kq[t]) + 1) & ~1;   // players of the round-robin
  const int npairs = np / 2;
  constexpr int JLD = jacobi_ld(RPL), ROWS = JPARTS * RPL;
  T *Ms = reinterpret_cast<T *>(jacobi_lds);
  T *Js = Ms + JLD * nall;
  const T *rt = R + (int64_t)t * n * n;
  for (int e = tid; e < ROWS * nall; e += CT) {
    const int r = e % ROWS, c = e / ROWS;
    Ms[r + c * JLD] = (r < n && c < n) ? rt[c + (int64_t)r * n] : T(0);    // M = R2^T
    Js[r + c * JLD] = r == c ? T(1) : T(0);
  }
  if (tid < 64) offw[tid / 32][tid % 32] = 0;
  __syncthreads();
  // thread (pair, part): pair jp = tid / 8 (CT / 8 = 32 pairs at most), rows
  // part, part + 8, ...  The eight lanes of a pair form its 2 x 2 Gram block,
  // each computes the rotation and applies it to its own rows: one barrier
  // per round (the next round pairs columns other waves wrote).
  const int jp = tid / JPARTS, jpart = tid % JPARTS;
  // Columns whose squared norm is below (n eps)^2 ||X||_F^2 are round-off:
  // they change no rank decision, and a pair holding one counts as
  // converged (rotating two such columns never reaches the cosine bound, so
  // every sweep would run).
  const T eps = sizeof(T) == 8 ? T(2.220446049250313e-16) : T(1.1920929e-7);
  const T negligible = (T(n) * eps) * (T(n) * eps) * norms2[t];
  int sweeps = 0, my_rot = 0;
  // the sweeps over the rows < 8 RP that a core can have nonzero (RP =
  // jacobi_rpl(np) for this tile: the rows from kq[t] on are zero in M and
  // in the columns of J that rotate), so a tile with a short basis does
  // proportionally less work per pair
  auto run = [&](auto rc) {
    constexpr int RP = decltype(rc)::value;
    for (int sweep = 0; sweep < 40 && np > 1; ++sweep) {
      ++sweeps;
      // round-robin: position 0 holds player 0, position x >= 1 player
      // 1 + (x - 1 + round) mod (np - 1), i.e. x at round 0, and each round
      // every player but 0 moves on by one (np - 1 wrapping to 1)
      int pa = jp, pb = np - 1 - jp;        // the players at this pair's two positions
      T cmax = 0;                            // this pair slot's largest cos^2 in the sweep
      for (int round = 0; round < np - 1; ++round) {
        if (jp < npairs) {
          const int p = min(pa, pb), q = max(pa, pb);
          // the pair's rows of M stay in registers for the rotation (its rows
          // of J are read only when it rotates: most pairs of a late sweep do not)
          T mp[RP], mq[RP];
          T al = 0, be = 0, ga = 0;
  #pragma unroll
          for (int e = 0; e < RP; ++e) {
            const int r = jpart + JPARTS * e;
            mp[e] = Ms[r + p * JLD];
            mq[e] = Ms[r + q * JLD];
            al += mp[e] * mp[e];
            be += mq[e] * mq[e];
            ga += mp[e] * mq[e];
          }
          static_assert(JPARTS == QRR_PARTS, "the 8-lane sums serve both kernels");
          al = part_sum8(al);
          be = part_sum8(be);
          ga = part_sum8(ga);
          // |cos| of the pair's angle against conv, squared (no square root);
          // the rotation's tangent tt = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)),
          // zeta = (be - al) / (2 ga), written with one division and one root
          const T g2 = ga * ga, ab = al * be;
          if (al > negligible && be > negligible && g2 > conv * conv * ab) {
            cmax = fmax(cmax, g2 / ab);
            if (jpart == 0) ++my_rot;
            const T d = be - al;
            const T sg = (d == T(0) || (d > T(0)) == (ga > T(0))) ? T(1) : T(-1);
            const T tt = sg * T(2) * fabs(ga) / (fabs(d) + sqrt(d * d + T(4) * g2));
            const T cs = T(1) / sqrt(T(1) + tt * tt);
            const T sn = cs * tt;
  #pragma unroll
            for (int e = 0; e < RP; ++e) {
              const int r = jpart + JPARTS * e;
              const T jpv = Js[r + p * JLD], jqv = Js[r + q * JLD];
              Ms[r + p * JLD] = cs * mp[e] - sn * mq[e];
              Ms[r + q * JLD] = sn * mp[e] + cs * mq[e];
              Js[r + p * JLD] = cs * jpv - sn * jqv;
              Js[r + q * JLD] = sn * jpv + cs * jqv;
            }
          }
          // the slot's maximum, before the sweep's last barrier; the buffers
          // alternate by sweep, so the next sweep's writes never meet this
          // sweep's reads
          if (jpart == 0 && round == np - 2) offw[sweep & 1][jp] = cmax;
        }
        if (pa != 0) pa = pa == np - 1 ? 1 : pa + 1;
        pb = pb == np - 1 ? 1 : pb + 1;
        __syncthreads();
      }
      // largest cos^2 of the sweep
      T mx = 0;
      for (int x = 0; x < npairs; ++x) mx = fmax(mx, offw[sweep & 1][x]);
      if (mx <= conv * conv) break;
    }
  };
  switch (jacobi_rpl(np)) {
    case 1: run(std::integral_constant<int, cmin(1, RPL)>()); break;
    case 2: run(std::integral_constant<int, cmin(2, RPL)>()); break;
    case 3: run(std::integral_constant<int, cmin(3, RPL)>()); break;
    case 4: run(std::integral_constant<int, cmin(4, RPL)>()); break;
    case 5: run(std::integral_constant<int, cmin(5, RPL)>()); break;
    case 6: run(std::integral_constant<int, cmin(6, RPL)>()); break;
    case 7: run(std::integral_constant<int, cmin(7, RPL)>()); break;
    default: run(std::integral_constant<int, RPL>()); break;
  }
  if (my_rot > 0) atomicAdd(&nrot, my_rot);   // LDS; read after the barriers below
  // column norms, the order of decreasing sigma (ties by column index)
  for (int c = wave; c < n; c += CT / 64) {
    T s = 0;
    for (int r = lane; r < nall; r += 64) s += Ms[r + c * JLD] * Ms[r + c * JLD];
    s = wave_sum(s);
    if (lane == 0) sig2[c] = s;
  }
  __syncthreads();
  for (int c = tid; c < n; c += CT) {
    int pos = 0;
    for (int d = 0; d < n; ++d) pos += (sig2[d] > sig2[c]) || (sig2[d] == sig2[c] && d < c);
    order[pos] = c;
  }
  __syncthreads();
  T *wt = Wout + (int64_t)t * n * n;
  T *jt = Jout + (int64_t)t * n * n;
  for (int e = tid; e < n * n; e += CT) {
    const int r = e % n, c = e / n;
    wt[e] = Ms[r + c * JLD];
    jt[e] = Js[r + c * JLD];
  }
  for (int c = tid; c < n; c += CT) perm[(int64_t)t * n + c] = order[c];
  if (tid == 0) {
    const T x2 = norms2[t];
    T captured = 0;
    for (int c = 0; c < n; ++c) captured += sig2[c];
    const T limit = tol * tol * x2;
    T tail = x2 > captured ? x2 - captured : T(0);
    int r = n;
    bool met = tail <= limit;
    if (met) {
      for (int pos = n - 1; pos >= 0; --pos) {
        const T s2 = sig2[order[pos]];
        if (tail + s2 <= limit) {
          tail += s2;
          r = pos;
        } else {
          break;
        }
      }
    }
    int fl = met ? 0 : 1;
    if (r > max_rank) {
      r = max_rank;
      fl = 1;
    }
    ranks[t] = r;
    flags[t] = fl;
    jstat[2 * t] = sweeps * npairs * (np - 1);
    jstat[2 * t + 1] = nrot;
  }
}

// Prefix sums of the ranks: outer offsets in tile-row order, inner offsets
// in tile-column order, each an exclusive scan over the q_r x q_c tiles in
// that order by the whole workgroup, SCAN_THREADS tiles at a time (wave scans
// by lane shuffles, then the wave totals).  info[0] = columns in all,
// info[1] = tiles flagged, info[2] = 1 when the columns exceed the capacity,
// info[3], info[4] = Jacobi pair visits and rotations summed over the tiles,
// info[5] = the sketch basis columns kept (kq) summed over the tiles.
constexpr int SCAN_THREADS = 256;

// exclusive prefix sum of v over the workgroup; *total = the sum of all v
// (in every thread)
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *wsum, int64_t *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < SCAN_THREADS / 64; ++k) {
    before += k < w ? wsum[k] : 0;
    all += wsum[k];
  }
  __syncthreads();   // wsum is written again by the next call
  *total = all;
  return before + x - v;
}

__device__ void offsets_by_rows_and_cols(const int32_t *ranks, int qr, int qc, int skip_diag, int64_t *ooff,
                                         int64_t *ioff, int64_t *total_out) {
  __shared__ int64_t wsum[SCAN_THREADS / 64];
  const int64_t nt = (int64_t)qr * qc;
  // outer: tile (i, j) after every tile of rows < i and tiles (i, j' < j)
  int64_t carry = 0;
  for (int64_t base = 0; base < nt; base += SCAN_THREADS) {
    const int64_t e = base + threadIdx.x;   // e = j + i qc
    const int i = e < nt ? (int)(e / qc) : 0, j = e < nt ? (int)(e % qc) : 0;
    const int64_t v = (e < nt && !(skip_diag && i == j)) ? ranks[i + (int64_t)j * qr] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan(v, wsum, &tot);
    if (e < nt) ooff[i + (int64_t)j * qr] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) *total_out = carry;
  // inner: tile (i, j) after every tile of columns < j and tiles (i' < i, j),
  // the storage order of the rank table
  carry = 0;
  for (int64_t base = 0; base < nt; base += SCAN_THREADS) {
    const int64_t e = base + threadIdx.x;   // e = i + j qr
    const int i = e < nt ? (int)(e % qr) : 0, j = e < nt ? (int)(e / qr) : 0;
    const int64_t v = (e < nt && !(skip_diag && i == j)) ? ranks[e] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan(v, wsum, &tot);
    if (e < nt) ioff[e] = carry + ex;
    carry += tot;
  }
  __syncthreads();   // *total_out is read by every thread after this
}

__global__ __launch_bounds__(SCAN_THREADS) void rank_scan_kernel(const int32_t *ranks, const int32_t *flags,
                                                                const int32_t *jstat, const int32_t *kq, int qr,
                                                                int qc, int skip_diag,
                                                                int64_t *ooff, int64_t *ioff, int64_t capacity,
                                                                int32_t *info) {
  __shared__ int64_t total;
  __shared__ int64_t part_w[4][SCAN_THREADS / 64];
  offsets_by_rows_and_cols(ranks, qr, qc, skip_diag, ooff, ioff, &total);
  int64_t nf = 0, nvis = 0, nrot = 0, nkq = 0;
  for (int t = threadIdx.x; t < qr * qc; t += SCAN_THREADS) {
    if (!(skip_diag && t % qr == t / qr)) {   // kq of a skipped tile is never written
      nf += flags[t];
      nkq += kq[t];
    }
    nvis += jstat[2 * t];
    nrot += jstat[2 * t + 1];
  }
  nf = wave_sum(nf);
  nvis = wave_sum(nvis);
  nrot = wave_sum(nrot);
  nkq = wave_sum(nkq);
  if ((threadIdx.x & 63) == 0) {
    part_w[0][threadIdx.x >> 6] = nf;
    part_w[1][threadIdx.x >> 6] = nvis;
    part_w[2][threadIdx.x >> 6] = nrot;
    part_w[3][threadIdx.x >> 6] = nkq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t x[4] = {0, 0, 0, 0};
    for (int k = 0; k < 4; ++k)
      for (int w = 0; w < SCAN_THREADS / 64; ++w) x[k] += part_w[k][w];
    info[0] = (int32_t)min<int64_t>(total, 0x7fffffff);
    info[1] = (int32_t)x[0];
    info[2] = total > capacity ? 1 : 0;
    info[3] = (int32_t)min<int64_t>(x[1], 0x7fffffff);
    info[4] = (int32_t)min<int64_t>(x[2], 0x7fffffff);
    info[5] = (int32_t)min<int64_t>(x[3], 0x7fffffff);
  }
}

// Packed output: kept column k of tile t goes to column ooff[t] + k of outer
// (U = Q W, the first s_i rows, leading dim b) and ioff[t] + k of inner
// (V = Q2 J, s_j rows); diagonal tiles are copied into their slots.  Nothing
// is written when the columns exceed the capacity.
template <typename T>
__global__ __launch_bounds__(CT) void pack_kernel(const T *X, int64_t ldx, const T *Uf, const T *Vf, int64_t fstride,
                                                 const int32_t *perm, const int32_t *ranks, const int64_t *ooff,
                                                 const int64_t *ioff, const int32_t *info, int qr, int qc,
                                                 int64_t rows, int64_t cols, int64_t b, int n, int has_diag,
                                                 T *outer, T *inner, T *diag, int32_t *ranks_out) {
  const int t = blockIdx.x;
  const int i = t % qr, j = t / qr;
  const int si = tile_rows(rows, b, i), sj = tile_rows(cols, b, j);
  if (has_diag && i == j) {
    if (threadIdx.x == 0) ranks_out[t] = 0;
    const T *x = X + (int64_t)i * b + (int64_t)j * b * ldx;
    T *d = diag + (int64_t)i * b * b;
    // eight elements per thread and step, loads first: eight in flight
    constexpr int PU = 8;
    for (int e0 = 0; e0 < si * si; e0 += PU * CT) {
      T v[PU];
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const int e = e0 + u * CT + threadIdx.x;
        v[u] = e < si * si ? x[e % si + (int64_t)(e / si) * ldx] : T(0);
      }
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const int e = e0 + u * CT + threadIdx.x;
        if (e < si * si) d[e % si + (int64_t)(e / si) * b] = v[u];
      }
    }
    return;
  }
  const int r = ranks[t];
  if (threadIdx.x == 0) ranks_out[t] = r;
  if (info[2]) return;
  const T *uf = Uf + (int64_t)t * fstride;
  const T *vf = Vf + (int64_t)t * fstride;
  // kept column k: U from column perm[k] of Uf, V from Vf; eight columns
  // per step, loads first
  constexpr int PK = 8;
  const int64_t o0 = ooff[t], i0 = ioff[t];
  for (int k0 = 0; k0 < r; k0 += PK) {
    for (int e = threadIdx.x; e < max(si, sj); e += CT) {
      T uv[PK], vv[PK];
#pragma unroll
      for (int u = 0; u < PK; ++u) {
        const int k = k0 + u;
        const int src = k < r ? perm[(int64_t)t * n + k] : 0;
        uv[u] = (k < r && e < si) ? uf[e + (int64_t)src * b] : T(0);
        vv[u] = (k < r && e < sj) ? vf[e + (int64_t)src * b] : T(0);
      }
#pragma unroll
      for (int u = 0; u < PK; ++u) {
        const int k = k0 + u;
        if (k < r && e < si) outer[(o0 + k) * b + e] = uv[u];
        if (k < r && e < sj) inner[(i0 + k) * b + e] = vv[u];
      }
    }
  }
}

// ---- expansion of a stored TLR operand --------------------------------------

// Column offsets of every tile's factors from the device rank table.
__global__ __launch_bounds__(SCAN_THREADS) void factor_offsets_kernel(const int32_t *ranks, int qr, int qc,
                                                                     int has_diag, int64_t *ooff, int64_t *ioff) {
  __shared__ int64_t total;
  offsets_by_rows_and_cols(ranks, qr, qc, has_diag, ooff, ioff, &total);
}

// C[64 x 64 block of tile t] <- alpha X_t + beta C (C read only when beta != 0):
// X_t = U V^T for an off-diagonal tile (rank-k chunks of 16 staged in LDS),
// the dense slot for a diagonal tile.
constexpr int EB = 64, EK = 16;
template <typename T>
__global__ __launch_bounds__(CT) void expand_kernel(const int32_t *ranks, const int64_t *ooff, const int64_t *ioff,
                                                   const T *outer, const T *inner, const T *diag, int qr, int qc,
                                                   int64_t rows, int64_t cols, int64_t b, int has_diag, T alpha,
                                                   T beta, T *C, int64_t ldc, int blocks_per_tile, int bpd) {
  __shared__ T Us[EK][EB + 1];
  __shared__ T Vs[EK][EB + 1];
  const int t = blockIdx.x / blocks_per_tile, blk = blockIdx.x - t * blocks_per_tile;
  const int i = t % qr, j = t / qr;
  const int si = tile_rows(rows, b, i), sj = tile_rows(cols, b, j);
  const int r0 = (blk % bpd) * EB, c0 = (blk / bpd) * EB;
  if (r0 >= si || c0 >= sj) return;
  const int tid = threadIdx.x;
  const int tr = tid % 16, tc = tid / 16;       // 4 x 4 outputs per thread: rows r0 + tr + 16a, cols c0 + tc + 16c
  T acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0;
  if (has_diag && i == j) {
    const T *d = diag + (int64_t)i * b * b;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int rr = r0 + tr + 16 * a, cc = c0 + tc + 16 * c;
        if (rr < si && cc < sj) acc[a][c] = d[rr + (int64_t)cc * b];
      }
  } else {
    const int rk = ranks[t];
    const T *u = outer + ooff[t] * b;
    const T *v = inner + ioff[t] * b;
    for (int k0 = 0; k0 < rk; k0 += EK) {
      __syncthreads();
      for (int e = tid; e < EK * EB; e += CT) {
        const int kk = e / EB, x = e % EB;
        const bool okk = k0 + kk < rk;
        Us[kk][x] = (okk && r0 + x < si) ? u[(int64_t)(k0 + kk) * b + r0 + x] : T(0);
        Vs[kk][x] = (okk && c0 + x < sj) ? v[(int64_t)(k0 + kk) * b + c0 + x] : T(0);
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < EK; ++kk)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[a][c] += Us[kk][tr + 16 * a] * Vs[kk][tc + 16 * c];
    }
  }
  const int64_t base = (int64_t)i * b + (int64_t)j * b * ldc;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int rr = r0 + tr + 16 * a, cc = c0 + tc + 16 * c;
      if (rr < si && cc < sj) {
        T *p = C + base + rr + (int64_t)cc * ldc;
        T y = alpha * acc[a][c];
        if (beta != T(0)) y += beta * *p;
        *p = y;
      }
    }
}

template <typename T>
T *as(void *p) { return static_cast<T *>(p); }

struct CompressLayout {
  int qr = 0, qc = 0, s = 0;
  int64_t ntile = 0;
  size_t y = 0, bt = 0, uf = 0, vf = 0, r2 = 0, w = 0, j = 0, norms = 0, perm = 0, ranks = 0, flags = 0, jstat = 0,
         kq = 0, ooff = 0, ioff = 0, total = 0;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

CompressLayout compress_layout(int64_t rows, int64_t cols, int64_t b, int max_rank, size_t es) {
  CompressLayout L;
  L.qr = (int)((rows + b - 1) / b);
  L.qc = (int)((cols + b - 1) / b);
  L.s = max_rank + OVERSAMPLE;
  L.ntile = (int64_t)L.qr * L.qc;
  const size_t panel = al256((size_t)L.ntile * b * L.s * es), core = al256((size_t)L.ntile * L.s * L.s * es);
  size_t o = 0;
  L.y = o; o += panel;
  L.bt = o; o += panel;
  L.uf = o; o += panel;
  L.vf = o; o += panel;
  L.r2 = o; o += core;
  L.w = o; o += core;
  L.j = o; o += core;
  L.norms = o; o += al256((size_t)L.ntile * es);
  L.perm = o; o += al256((size_t)L.ntile * L.s * 4);
  L.ranks = o; o += al256((size_t)L.ntile * 4);
  L.flags = o; o += al256((size_t)L.ntile * 4);
  L.jstat = o; o += al256((size_t)L.ntile * 8);
  L.kq = o; o += al256((size_t)L.ntile * 4);
  L.ooff = o; o += al256((size_t)L.ntile * 8);
  L.ioff = o; o += al256((size_t)L.ntile * 8);
  L.total = o;
  return L;
}

tlr_status check_compress_args(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t max_rank) {
  if (dt == TLR_F16 || dt == TLR_BF16) return fail(TLR_ERR_UNSUPPORTED, "compress: 16-bit types are not provided");
  if (dt != TLR_F32 && dt != TLR_F64) return fail(TLR_ERR_INVALID_ARG, "compress: bad dtype");
  if (rows < 0 || cols < 0 || b < 1) return fail(TLR_ERR_INVALID_ARG, "compress: bad dimensions or tile size");
  if (rows > 0x7fffffff || cols > 0x7fffffff || b > 4096) return fail(TLR_ERR_INVALID_ARG, "compress: dimensions too large");
  if (max_rank < 0 || max_rank + OVERSAMPLE > S_MAX)
    return fail(TLR_ERR_UNSUPPORTED, "compress: max_rank must lie in [0, " + std::to_string(S_MAX - OVERSAMPLE) + "]");
  return TLR_OK;
}

// The Jacobi sweeps stop once no pair's |cos| exceeds this bound.  The column
// norms then equal the singular values to about bound^2 relative (the Gram
// matrix's off-diagonal part moves its eigenvalues only to second order):
// 1e-16 for fp64, its rounding, and 1e-10 for fp32, below its rounding.  The
// truncation error itself is exact whatever the bound, since W J^T = M with J
// orthogonal: dropping columns of W drops exactly their norms.
template <typename T>
T conv_tol() { return sizeof(T) == 8 ? T(1e-8) : T(1e-5f); }

// The early stop of the QR of the sketches: the basis stops growing once the
// sketch puts the energy it leaves out near 1e-10 tol^2 ||X||_F^2, below
// 1e-7 tol^2 ||X||_F^2 with probability above 1 - 1e-11.  That changes the
// discarded energy the rank decision sees by at most 1e-7 of its bound and
// the result tile by at most about 3e-4 tol ||X||_F.
template <typename T>
T range_stop(double tol) { return (T)(1e-10 * tol * tol); }

// One launch of the Jacobi kernel for RPL rows per lane; the widest sketch
// (S_MAX columns, RPL = 8) needs more than the default 64 KB of dynamic LDS
// in fp64, which is raised once per instantiation.
template <typename T, int RPL, typename... Args>
tlr_status launch_jacobi(int64_t nt, int np, hipStream_t s, Args... args) {
  const size_t lds = 2 * (size_t)np * jacobi_ld(RPL) * sizeof(T);
  if (lds > 65536) {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
      err = hipFuncSetAttribute(reinterpret_cast<const void *>(&jacobi_rank_kernel<T, RPL>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)(2 * JPARTS * RPL * jacobi_ld(RPL) * sizeof(T)));
    });
    if (err != hipSuccess)
      return fail(TLR_ERR_HIP, std::string("Jacobi SVD LDS attribute: ") + hipGetErrorString(err));
  }
  hipLaunchKernelGGL((jacobi_rank_kernel<T, RPL>), dim3((unsigned)nt), dim3(CT), lds, s, args...);
  return TLR_OK;
}

// Optional event pairs around the kernel groups of a compression
// (tlr_compress_profile): 0 tile norms, 1 sketch product, 2 QR of the
// sketches, 3 projection product, 4 QR of the projections, 5 Jacobi SVD and
// ranks, 6 factor products, 7 rank scan, 8 packing.
struct CompressProfile {
  std::mutex mu;
  int remaining = 0;   // calls still to record
  int calls = 0;       // calls recorded since the last read
  struct Rec {
    int group;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
};
CompressProfile &cprof() {
  static CompressProfile p;
  return p;
}

// Events of one call: begin(g) records the start of group g, end() its end.
struct ProfileMarks {
  bool on = false;
  hipStream_t s = nullptr;
  std::vector<CompressProfile::Rec> recs;
  bool begin(int group) {
    if (!on) return true;
    CompressProfile::Rec r{group, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess) return false;
    if (hipEventCreate(&r.b) != hipSuccess) {
      (void)hipEventDestroy(r.a);
      return false;
    }
    recs.push_back(r);
    return hipEventRecord(r.a, s) == hipSuccess;
  }
  bool end() {
    if (!on) return true;
    if (hipEventRecord(recs.back().b, s) != hipSuccess) return false;
    ++ended;
    return true;
  }
  size_t ended = 0;   // leading records whose end event was recorded
  ~ProfileMarks() {   // hand the complete pairs to the record; a call that failed midway leaves the rest
    if (!on) return;
    CompressProfile &p = cprof();
    std::lock_guard<std::mutex> g(p.mu);
    for (size_t k = 0; k < recs.size(); ++k) {
      if (k < ended) {
        p.recs.push_back(recs[k]);
      } else {
        (void)hipEventDestroy(recs[k].a);
        (void)hipEventDestroy(recs[k].b);
      }
    }
  }
};

#define CHECK_LAUNCH(what)                                                                     \
  do {                                                                                         \
    hipError_t e_ = hipGetLastError();                                                         \
    if (e_ != hipSuccess) return fail(TLR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e_)); \
  } while (0)

template <typename T>
tlr_status compress_t(int64_t rows, int64_t cols, int64_t b, int has_diag, const void *X, int64_t ldx, double tol,
                      int max_rank, const void *omega, int32_t *ranks_out, void *diag, void *outer, void *inner,
                      int64_t capacity, int32_t *info, void *ws, const CompressLayout &L, hipStream_t s) {
  const tlr_dtype dt = sizeof(T) == 8 ? TLR_F64 : TLR_F32;
  char *w = static_cast<char *>(ws);
  const int n = L.s;
  const int nt = (int)L.ntile;
  const int skip = has_diag ? 1 : 0;
  ProfileMarks pm;
  pm.s = s;
  {
    CompressProfile &p = cprof();
    std::lock_guard<std::mutex> g(p.mu);
    if (p.remaining > 0) {
      --p.remaining;
      ++p.calls;
      pm.on = true;
    }
  }
#define MARK(call)                                                                  \
  do {                                                                              \
    if (!(call)) return fail(TLR_ERR_HIP, "compress: profiling event failed");     \
  } while (0)
  T *norms = as<T>(w + L.norms);
  MARK(pm.begin(0));
  hipLaunchKernelGGL(tile_norms_kernel<T>, dim3(nt), dim3(CT), 0, s, static_cast<const T *>(X), ldx, L.qr, L.qc, rows,
                     cols, b, norms);
  CHECK_LAUNCH("tile norms");
  MARK(pm.end());
  Bases bases;
  for (auto &p : bases.p) p = nullptr;
  bases.p[BASE_A_OUTER] = X;
  bases.p[BASE_B_OUTER] = omega;
  bases.p[BASE_WS] = ws;
  const int64_t es = sizeof(T);
  auto wsoff = [&](size_t byte_off) { return (int64_t)(byte_off / es); };
  const int64_t panel = b * n;   // elements per tile of a b x s panel
  auto ta = [](int64_t off, int64_t f_ro, int64_t f_co, int64_t f_t, int64_t ld, uint8_t base, uint8_t trans) {
    TileAddr a;
    a.off = off; a.f_ro = f_ro; a.f_co = f_co; a.f_t = f_t; a.ld = (int32_t)ld; a.base = base; a.trans = trans;
    return a;
  };
  auto gemm = [&](int m_sel, int k_sel, TileAddr A, TileAddr B, TileAddr C, int mode) -> tlr_status {
    TileGemm g;
    g.qr = L.qr; g.qc = L.qc; g.rows = rows; g.cols = cols; g.b = b; g.skip_diag = skip;
    g.m_sel = m_sel; g.k_sel = k_sel; g.n = n; g.n_fixed = n;
    g.a = A; g.bop = B; g.c = C;
    const int e = launch_tile_gemm(dt, mode, g, bases, s);
    if (e) return fail(TLR_ERR_HIP, std::string("tile GEMM launch: ") + hipGetErrorString((hipError_t)e));
    return TLR_OK;
  };
  // pair loads need even sizes, offsets and leading dimensions throughout
  const bool even = b % 2 == 0 && rows % 2 == 0 && cols % 2 == 0 && ldx % 2 == 0 && n % 2 == 0 &&
                    reinterpret_cast<uintptr_t>(X) % (2 * es) == 0 && reinterpret_cast<uintptr_t>(omega) % (2 * es) == 0;
  // 1. Y_t = X_t Omega                       (s_i x s)
  MARK(pm.begin(1));
  tlr_status st = gemm(0, 1, ta(0, 1, ldx, 0, ldx, BASE_A_OUTER, 0), ta(0, 0, 0, 0, b, BASE_B_OUTER, 0),
                       ta(wsoff(L.y), 0, 0, panel, b, BASE_WS, 0), even ? LOAD_PAIR_M : LOAD_SINGLE);
  if (st != TLR_OK) return st;
  MARK(pm.end());
  // 2. Y_t = Q R, Q kept in place
  int32_t *kq = as<int32_t>(w + L.kq);
  auto qr_launch = [&](T *A, T *R, int m_sel, int kq_mode) {
    if (b <= QR_ROWS && n <= S_MAX)
      hipLaunchKernelGGL((qr_reg_kernel<T>), dim3(nt), dim3(QRR_THREADS), 0, s, A, (int)b, panel, R, L.qr, L.qc,
                         rows, cols, b, m_sel, n, skip, kq, kq_mode, (const T *)norms, range_stop<T>(tol));
    else
      hipLaunchKernelGGL((qr_tiles_kernel<T>), dim3(nt), dim3(CT), 0, s, A, (int)b, panel, R, L.qr, L.qc, rows,
                         cols, b, m_sel, n, skip, kq, kq_mode);
  };
  MARK(pm.begin(2));
  qr_launch(as<T>(w + L.y), (T *)nullptr, 0, KQ_SET);
  CHECK_LAUNCH("QR of the sketches");
  MARK(pm.end());
  // 3. Bt_t = X_t^T Q_t                      (s_j x s)
  MARK(pm.begin(3));
  st = gemm(1, 0, ta(0, 1, ldx, 0, ldx, BASE_A_OUTER, 1), ta(wsoff(L.y), 0, 0, panel, b, BASE_WS, 0),
            ta(wsoff(L.bt), 0, 0, panel, b, BASE_WS, 0), even ? LOAD_PAIR_K : LOAD_SINGLE);
  if (st != TLR_OK) return st;
  MARK(pm.end());
  // 4. Bt_t = Q2 R2
  MARK(pm.begin(4));
  qr_launch(as<T>(w + L.bt), as<T>(w + L.r2), 1, KQ_CAP);
  CHECK_LAUNCH("QR of the projections");
  MARK(pm.end());
  // 5. Jacobi on M = R2^T, ranks
  MARK(pm.begin(5));
  const int jnp = (n + 1) & ~1;
  {
    tlr_status js = TLR_OK;
    auto jac = [&](auto rc) {
      constexpr int RPL = decltype(rc)::value;
      js = launch_jacobi<T, RPL>(nt, jnp, s, as<T>(w + L.r2), as<T>(w + L.w), as<T>(w + L.j),
                                 as<int32_t>(w + L.perm), as<int32_t>(w + L.ranks), as<int32_t>(w + L.flags),
                                 as<int32_t>(w + L.jstat), norms, (const int32_t *)kq, L.qr, L.qc, n, max_rank,
                                 (T)tol, conv_tol<T>(), skip);
    };
    switch (jacobi_rpl(jnp)) {
      case 1: jac(std::integral_constant<int, 1>()); break;
      case 2: jac(std::integral_constant<int, 2>()); break;
      case 3: jac(std::integral_constant<int, 3>()); break;
      case 4: jac(std::integral_constant<int, 4>()); break;
      case 5: jac(std::integral_constant<int, 5>()); break;
      case 6: jac(std::integral_constant<int, 6>()); break;
      case 7: jac(std::integral_constant<int, 7>()); break;
      default: jac(std::integral_constant<int, 8>()); break;
    }
    if (js != TLR_OK) return js;
  }
  CHECK_LAUNCH("Jacobi SVD");
  MARK(pm.end());
  // 6. U_t = Q_t W_t, V_t = Q2_t J_t        (s_i x s, s_j x s)
  MARK(pm.begin(6));
  st = gemm(0, 2, ta(wsoff(L.y), 0, 0, panel, b, BASE_WS, 0), ta(wsoff(L.w), 0, 0, (int64_t)n * n, n, BASE_WS, 0),
            ta(wsoff(L.uf), 0, 0, panel, b, BASE_WS, 0), even ? LOAD_PAIR_M : LOAD_SINGLE);
  if (st != TLR_OK) return st;
  st = gemm(1, 2, ta(wsoff(L.bt), 0, 0, panel, b, BASE_WS, 0), ta(wsoff(L.j), 0, 0, (int64_t)n * n, n, BASE_WS, 0),
            ta(wsoff(L.vf), 0, 0, panel, b, BASE_WS, 0), even ? LOAD_PAIR_M : LOAD_SINGLE);
  if (st != TLR_OK) return st;
  MARK(pm.end());
  // 7. offsets, 8. packed factors and diagonal slots
  MARK(pm.begin(7));
  hipLaunchKernelGGL(rank_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, as<int32_t>(w + L.ranks),
                     as<int32_t>(w + L.flags), as<int32_t>(w + L.jstat), (const int32_t *)kq, L.qr, L.qc, skip,
                     as<int64_t>(w + L.ooff), as<int64_t>(w + L.ioff),
                     capacity, info);
  CHECK_LAUNCH("rank scan");
  MARK(pm.end());
  MARK(pm.begin(8));
  hipLaunchKernelGGL(pack_kernel<T>, dim3(nt), dim3(CT), 0, s, static_cast<const T *>(X), ldx, as<T>(w + L.uf),
                     as<T>(w + L.vf), panel, as<int32_t>(w + L.perm), as<int32_t>(w + L.ranks),
                     as<int64_t>(w + L.ooff), as<int64_t>(w + L.ioff), info, L.qr, L.qc, rows, cols, b, n, skip,
                     static_cast<T *>(outer), static_cast<T *>(inner), static_cast<T *>(diag), ranks_out);
  CHECK_LAUNCH("pack");
  MARK(pm.end());
#undef MARK
  return TLR_OK;
}

template <typename T>
tlr_status expand_t(int64_t rows, int64_t cols, int64_t b, int has_diag, const int32_t *ranks, const tlr_buffers *X,
                    double alpha, double beta, void *C, int64_t ldc, void *ws, hipStream_t s) {
  const int qr = (int)((rows + b - 1) / b), qc = (int)((cols + b - 1) / b);
  const int64_t nt = (int64_t)qr * qc;
  int64_t *ooff = static_cast<int64_t *>(ws);
  int64_t *ioff = ooff + nt;
  hipLaunchKernelGGL(factor_offsets_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, ranks, qr, qc, has_diag, ooff, ioff);
  CHECK_LAUNCH("factor offsets");
  const int bpd = (int)((b + EB - 1) / EB);
  const int bpt = bpd * bpd;
  hipLaunchKernelGGL(expand_kernel<T>, dim3((unsigned)(nt * bpt)), dim3(CT), 0, s, ranks, ooff, ioff,
                     static_cast<const T *>(X->outer), static_cast<const T *>(X->inner),
                     static_cast<const T *>(X->diag), qr, qc, rows, cols, b, has_diag, (T)alpha, (T)beta,
                     static_cast<T *>(C), ldc, bpt, bpd);
  CHECK_LAUNCH("expand");
  return TLR_OK;
}

}  // namespace

tlr_status compress_workspace(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t max_rank, size_t *bytes) {
  if (!bytes) return fail(TLR_ERR_INVALID_ARG, "compress: null output");
  tlr_status st = check_compress_args(dt, rows, cols, b, max_rank);
  if (st != TLR_OK) return st;
  *bytes = compress_layout(rows, cols, b, max_rank, dt == TLR_F64 ? 8 : 4).total;
  return TLR_OK;
}

tlr_status compress(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag, const void *X, int64_t ldx,
                    double tol, int32_t max_rank, const void *omega, int32_t *ranks_out, void *diag, void *outer,
                    void *inner, int64_t capacity, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  tlr_status st = check_compress_args(dt, rows, cols, b, max_rank);
  if (st != TLR_OK) return st;
  if (has_diag && rows != cols) return fail(TLR_ERR_INVALID_ARG, "compress: a dense diagonal needs a square matrix");
  if (!(tol >= 0.0)) return fail(TLR_ERR_INVALID_ARG, "compress: tolerance must be >= 0");
  if (ldx < std::max<int64_t>(1, rows) || ldx >= ((int64_t)1 << 21))
    return fail(TLR_ERR_INVALID_ARG, "compress: ldx must lie in [rows, 2^21)");
  if (capacity < 0) return fail(TLR_ERR_INVALID_ARG, "compress: negative capacity");
  if (rows == 0 || cols == 0) return TLR_OK;
  const size_t es = dt == TLR_F64 ? 8 : 4;
  const CompressLayout L = compress_layout(rows, cols, b, max_rank, es);
  if (!X || !omega || !ranks_out || !info || !ws || (has_diag && !diag) || (capacity > 0 && (!outer || !inner)))
    return fail(TLR_ERR_INVALID_ARG, "compress: null buffer");
  if (ws_bytes < L.total) return fail(TLR_ERR_WORKSPACE, "compress: workspace smaller than tlr_compress_workspace_bytes");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(TLR_ERR_INVALID_ARG, "compress: workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F64)
    return compress_t<double>(rows, cols, b, has_diag, X, ldx, tol, max_rank, omega, ranks_out, diag, outer, inner,
                              capacity, info, ws, L, s);
  return compress_t<float>(rows, cols, b, has_diag, X, ldx, tol, max_rank, omega, ranks_out, diag, outer, inner,
                           capacity, info, ws, L, s);
}

tlr_status compress_profile(int32_t max_calls) {
  if (max_calls < 0) return fail(TLR_ERR_INVALID_ARG, "compress profile: negative call count");
  CompressProfile &p = cprof();
  std::lock_guard<std::mutex> g(p.mu);
  p.remaining = max_calls;
  return TLR_OK;
}

tlr_status compress_profile_read(double *group_ms, int32_t *calls) {
  if (!group_ms || !calls) return fail(TLR_ERR_INVALID_ARG, "compress profile: null output");
  CompressProfile &p = cprof();
  std::lock_guard<std::mutex> g(p.mu);
  for (int k = 0; k < COMPRESS_PROFILE_GROUPS; ++k) group_ms[k] = 0.0;
  tlr_status st = TLR_OK;
  for (const CompressProfile::Rec &r : p.recs) {
    float ms = 0.0f;
    if (st == TLR_OK && hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = fail(TLR_ERR_HIP, "compress profile: events not complete (synchronise first)");
    if (st == TLR_OK && r.group >= 0 && r.group < COMPRESS_PROFILE_GROUPS) group_ms[r.group] += ms;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  *calls = p.calls;
  p.recs.clear();
  p.calls = 0;
  return st;
}

tlr_status expand(tlr_dtype dt, int64_t rows, int64_t cols, int32_t b, int32_t has_diag, const int32_t *ranks,
                  const tlr_buffers *X, double alpha, double beta, void *C, int64_t ldc, void *ws, size_t ws_bytes,
                  void *stream) {
  if (dt == TLR_F16 || dt == TLR_BF16) return fail(TLR_ERR_UNSUPPORTED, "expand: 16-bit types are not provided");
  if (dt != TLR_F32 && dt != TLR_F64) return fail(TLR_ERR_INVALID_ARG, "expand: bad dtype");
  if (rows < 0 || cols < 0 || b < 1) return fail(TLR_ERR_INVALID_ARG, "expand: bad dimensions or tile size");
  if (has_diag && rows != cols) return fail(TLR_ERR_INVALID_ARG, "expand: a dense diagonal needs a square matrix");
  if (ldc < std::max<int64_t>(1, rows)) return fail(TLR_ERR_INVALID_ARG, "expand: ldc smaller than rows");
  if (rows == 0 || cols == 0) return TLR_OK;
  if (!C || !X || !ranks || !ws) return fail(TLR_ERR_INVALID_ARG, "expand: null buffer");
  if (has_diag && !X->diag) return fail(TLR_ERR_INVALID_ARG, "expand: null diagonal");
  const int64_t qrr = (rows + b - 1) / b, qcc = (cols + b - 1) / b, nt = qrr * qcc;
  if (ws_bytes < (size_t)(16 * nt)) return fail(TLR_ERR_WORKSPACE, "expand: workspace below 16 bytes per tile");
  if (reinterpret_cast<uintptr_t>(ws) % 8) return fail(TLR_ERR_INVALID_ARG, "expand: workspace not 8-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F64) return expand_t<double>(rows, cols, b, has_diag, ranks, X, alpha, beta, C, ldc, ws, s);
  return expand_t<float>(rows, cols, b, has_diag, ranks, X, alpha, beta, C, ldc, ws, s);
}

}  // namespace tlr
