// Grouped, segmented-K MFMA GEMM for gfx950 (CDNA4), IEEE half and bfloat16.
//
// The same task tables as the 32/64-bit kernel (tlr_desc.h): each workgroup
// reads one entry (task, m0, n0) and computes a 128 x BN block of that task's
// output (BN = 128 or 64, chosen per launch; the final update and other
// launches large enough use a second kernel with 256 x 256 blocks, further
// down), accumulating over the task's K
// segments in float with v_mfma_f32_16x16x32_{f16,bf16}, then writes
// C = alpha*acc + beta*C (final update) or C = acc (workspace intermediates),
// rounded once to the 16-bit type.
//
// Every extent, offset and leading dimension is a multiple of 8 (the host
// enforces it: stored ranks rounded up to a multiple of 8), so operands move
// in 16-byte vectors of 8 elements along their contiguous index and a vector
// lies wholly inside or wholly outside its operand.
//
// The 16-bit matrix cores take, per lane, 8 consecutive k of one row of A and
// of one column of B.  Both operands therefore pass through LDS stored
// K-contiguous: [row][k] for A, [column][k] for B, rows of 32 k padded to 40
// elements (80 bytes: 8 consecutive rows start on 8 different 16-byte bank
// groups).  A stage (32 k) is cut into units of four 16-byte vectors, one per
// thread (waves 0-1: the A tile, waves 2-3: the B tile).  An operand that is
// K-contiguous in memory gives units of 4 rows x 8 k whose row pieces go to
// LDS as they are; an M- (or N-) contiguous one gives units of 8 rows x 4 k,
// transposed in registers (v_perm_b32) into eight 8-byte LDS stores.
//
// Work split: four wave64s in a 2 x 2 grid, each owning a 64 x BN/2 strip of
// the block as 4 x (BN/32) MFMA tiles of 16 x 16.  LDS holds two stages; the
// global loads of stage s+1 are in flight while stage s's MFMAs run, and one
// barrier per stage separates the LDS stores from the next reads.  Short
// stages and small units keep LDS at 40 KB and registers at 128 per lane, so
// four workgroups share a CU and overlap each other's barrier-separated
// phases (the lane's output column offsets go to scratch around the K loop).
// Measured on the final update: MFMA time is hidden entirely; LDS traffic and
// the per-stage barriers set the pace.  Against this form, two loading waves
// with 8-vector units (three workgroups per CU) were 12% slower, stages of
// 64 k (two workgroups per CU) 30% slower, and loading two stages ahead or
// reading fragments a k-step ahead slower still.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tlr_plan.h"

namespace tlr {

namespace {

constexpr int BM16 = 128;        // block rows
constexpr int KS = 32;           // k per stage
constexpr int LROW = 40;         // LDS row stride in elements (32 k + 8)
constexpr int NT16 = 256;        // four wave64s

template <int NJ> struct Blk16 {
  static constexpr int BN = 32 * NJ;   // block columns: two waves along N, NJ 16-column tiles each
};

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// H: _Float16 or __bf16.  mma: one 16 x 16 x 32 product; lane l supplies
// A[l % 16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l % 16] (any fixed
// assignment of the 32 k to lanes gives the same sum, provided A and B use
// the same one), and holds D[4*(l/16) + v][l % 16] in element v afterwards.
template <typename H> struct M16;
template <> struct M16<_Float16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f4 mma(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};
template <> struct M16<__bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f4 mma(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};

constexpr uint32_t OOB16 = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc16(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7fffffff, 0x00020000);
}

// LDS row of block row m in the A tile.  After the MFMAs, lane (r, g) of
// tile i = 2h + p holds rows 4g .. 4g+3 of that tile; the A rows are placed so
// that those are block rows 64w + 32h + 8g + 4p + v: the lane then holds the 8
// consecutive rows 64w + 32h + 8g .. +7 of each column, one 16-byte unit of C.
// In bits: m = [w h | g g | p | v v] sits at LDS row [w h | p | g g | v v].
__device__ __forceinline__ int a_lds_row(int m) { return (m & ~0x1C) | ((m & 0x4) << 2) | ((m & 0x18) >> 1); }

// One operand tile of a stage as seen by one loading thread (rows of the A
// tile, or columns of the B tile).  With kc (K-contiguous) vector e is row
// s0+e at k c0 .. c0+7; otherwise it is k s0+e at rows c0 .. c0+7.  Vector e
// sits e*ld elements past vector 0; that step goes into the lane's offset
// (given to the scalar offset instead, the compiler held it in vector
// registers inside the K loop and wrapped every load in a loop over distinct
// lane values).
struct Unit {
  const uint16_t *base;   // operand at (row 0 of the block, k 0)
  int64_t kstep;          // elements per stage along k
  uint32_t lane;          // byte offset of the thread's vector 0
  uint32_t ldb;           // leading dimension in bytes
  int s0, s_lim, c0, c_lim;   // strided / contiguous index of vector 0 and their limits
  bool kc;
};

__device__ __forceinline__ void load_unit(const Unit &u, int st, int krem, u4 (&x)[4]) {
  const __amdgpu_buffer_rsrc_t rs = rsrc16(u.base + (int64_t)st * u.kstep);
  // k limit of this stage: contiguous index for kc, strided otherwise
  const int s_lim = u.kc ? u.s_lim : krem, c_lim = u.kc ? krem : u.c_lim;
  const bool cok = u.c0 < c_lim;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = cok && u.s0 + e < s_lim;
    x[e] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? u.lane + e * u.ldb : OOB16, 0, 0));
  }
}

// LDS stores of a unit.  K-contiguous (kc): vector e is row 4a+e at k
// 8b..8b+7, stored as it is.  Otherwise vector e is k 4b+e at rows
// 8a..8a+7; transposed, row 8a+c gets k 4b..4b+3 (8 bytes).
template <bool IS_A>
__device__ __forceinline__ void store_unit(uint16_t *tile, int a, int b, bool kc, const u4 (&x)[4]) {
  if (kc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = IS_A ? a_lds_row(4 * a + e) : 4 * a + e;
      *reinterpret_cast<u4 *>(tile + row * LROW + 8 * b) = x[e];
    }
  } else {
    // dword w of a vector holds elements 2w (low half) and 2w+1 (high half);
    // v_perm_b32 takes bytes 0-3 from its second source and 4-7 from its
    // first: selector 0x05040100 packs the two low halves, 0x07060302 the
    // two high halves
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u2 y;
      y[0] = __builtin_amdgcn_perm(x[1][c >> 1], x[0][c >> 1], sel);
      y[1] = __builtin_amdgcn_perm(x[3][c >> 1], x[2][c >> 1], sel);
      const int row = IS_A ? a_lds_row(8 * a + c) : 8 * a + c;
      *reinterpret_cast<u2 *>(tile + row * LROW + 4 * b) = y;
    }
  }
}

template <typename H> __device__ __forceinline__ float to_f(uint16_t v) {
  return (float)__builtin_bit_cast(H, v);
}
template <typename H> __device__ __forceinline__ uint16_t from_f(float v) {
  return __builtin_bit_cast(uint16_t, (H)v);
}

template <typename H, int NJ>
__device__ __forceinline__ void gemm_block16(const DevTask &t, int m0, int n0, const int64_t *coltab,
                                             const Bases &bases, float alpha, float beta, float cscale) {
  constexpr int BN = Blk16<NJ>::BN;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM16 * LROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LROW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const int M = t.M, N = t.N;

  uint16_t *C = static_cast<uint16_t *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;
  const bool fin = t.final_ != 0;
  const bool preload = fin && cscale != 0.0f;
  const bool rd = fin && beta != 0.0f && !preload;

  // output columns of the lane (every column offset a multiple of 8 elements)
  int64_t ocol[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn * 16 * NJ + 16 * j + r;
    ocol[j] = n >= N ? 0 : (t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n]);
  }
  f4 acc[4][NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn * 16 * NJ + 16 * j + r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      acc[2 * h][j] = f4{0, 0, 0, 0};
      acc[2 * h + 1][j] = f4{0, 0, 0, 0};
      const int m = m0 + 64 * wm + 32 * h + 8 * g;
      if (preload && n < N && m < M) {
        const u4 x = *reinterpret_cast<const u4 *>(C + ocol[j] + m);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[2 * h + (e >> 2)][j][e & 3] = cscale * to_f<H>((uint16_t)(x[e >> 1] >> (16 * (e & 1))));
      }
    }
  }

  // loading role: waves 0-1 the A tile (128 units), waves 2-3 the B tile (BN
  // units: both waves, or wave 2 alone for BN = 64)
  const bool loads_a = wave < 2;
  const int uidx = loads_a ? tid : tid - 128;
  const bool has_unit = loads_a || (wave - 2) * 64 < BN;

  for (int sidx = 0; sidx < t.nseg; ++sidx) {
    const DevSeg &d = t.seg[sidx];
    const int K = d.K;
    if (K <= 0) continue;
    const int nst = (K + KS - 1) / KS;
    // operand of this thread's unit
    Unit u;
    {
      const DevOperand &o = loads_a ? d.a : d.b;
      const uint16_t *p = static_cast<const uint16_t *>(bases.p[o.base]) + o.off;
      const int64_t ld = o.ld;
      // A: trans 1 = K-contiguous; B: trans 0 = K-contiguous
      u.kc = loads_a ? o.trans == 1 : o.trans == 0;
      const int first = loads_a ? m0 : n0;
      const int rem = loads_a ? M - m0 : N - n0;
      u.base = u.kc ? p + (int64_t)first * ld : p + first;
      u.kstep = u.kc ? KS : (int64_t)KS * ld;
      u.ldb = (uint32_t)(ld * 2);
      // kc: rows 4rq.. (rq = uidx/4) at k chunk uidx%4; else k 4kq.. (kq = uidx%8) at rows 8rg.. (rg = uidx/8)
      const int srow = u.kc ? 4 * (uidx >> 2) : 4 * (uidx & 7), ccol = u.kc ? 8 * (uidx & 3) : 8 * (uidx >> 3);
      u.lane = (uint32_t)((int64_t)srow * ld + ccol) * 2u;
      u.s0 = srow;
      u.c0 = ccol;
      u.s_lim = u.kc ? rem : 0;   // the k limit is filled in per stage
      u.c_lim = u.kc ? 0 : rem;
    }
    u4 x[4];
    const int ua = u.kc ? uidx >> 2 : uidx >> 3, ub = u.kc ? uidx & 3 : uidx & 7;
    if (has_unit) {
      load_unit(u, 0, K, x);
      if (loads_a) store_unit<true>(As[0], ua, ub, u.kc, x);
      else store_unit<false>(Bs[0], ua, ub, u.kc, x);
    }
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const bool more = st + 1 < nst;
      if (more && has_unit) load_unit(u, st + 1, K - (st + 1) * KS, x);
      // one MFMA k-step of 32 per stage
      const uint16_t *a_t = As[st & 1];
      const uint16_t *b_t = Bs[st & 1];
      u4 af[4], bf[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u4 *>(a_t + (64 * wm + 16 * i + r) * LROW + 8 * g);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bf[j] = *reinterpret_cast<const u4 *>(b_t + (wn * 16 * NJ + 16 * j + r) * LROW + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = M16<H>::mma(af[i], bf[j], acc[i][j]);
      if (more && has_unit) {
        if (loads_a) store_unit<true>(As[(st + 1) & 1], ua, ub, u.kc, x);
        else store_unit<false>(Bs[(st + 1) & 1], ua, ub, u.kc, x);
      }
      __syncthreads();
    }
  }

  // epilogue: lane (r, g) holds rows 64wm + 32h + 8g .. +7 of each of its columns
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn * 16 * NJ + 16 * j + r;
    if (n >= N) continue;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + 64 * wm + 32 * h + 8 * g;
      if (m >= M) continue;
      u4 *q = reinterpret_cast<u4 *>(C + ocol[j] + m);
      u4 old = u4{0, 0, 0, 0};
      if (rd) old = *q;
      u4 y;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float v0 = acc[2 * h + (w >> 1)][j][2 * (w & 1)];
        float v1 = acc[2 * h + (w >> 1)][j][2 * (w & 1) + 1];
        if (fin) {
          v0 *= alpha;
          v1 *= alpha;
          if (rd) {
            v0 += beta * to_f<H>((uint16_t)(old[w] & 0xffffu));
            v1 += beta * to_f<H>((uint16_t)(old[w] >> 16));
          }
        }
        y[w] = (uint32_t)from_f<H>(v0) | ((uint32_t)from_f<H>(v1) << 16);
      }
      *q = y;
    }
  }
}

// ---- strips of the right/left product ------------------------------------
//
// A right/left-product task of K <= 32 (one k-step of the 16-bit MFMA) does a
// few MFMAs per 128 x 128 block and then stores it, so block overheads (the
// task read, the operand fetch and its latency) sit in front of every 32 KB
// of stores.  A strip block covers 128 rows and STRIP_W = 512 columns: the A
// tile (128 x 32) and the B strip (32 x 512) go to LDS once, as in
// gemm_block16 (K-contiguous rows, A rows placed by a_lds_row), then four
// 128-column chunks run back to back, each 16 MFMAs per wave followed by its
// stores in gemm_block16's epilogue layout, with no barrier between chunks.
// 50 KB of LDS: three workgroups per CU.
template <typename H>
__global__ __launch_bounds__(NT16) __attribute__((amdgpu_waves_per_eu(3)))
void strip_gemm16_kernel(const DevTask *__restrict__ tasks, const DevTile *__restrict__ tiles,
                         const int64_t *__restrict__ coltab, Bases bases) {
  constexpr int NJ = 4, BN = Blk16<NJ>::BN;   // a chunk: two waves along N, 4 tiles of 16 columns each
  static_assert(STRIP_W % BN == 0 && STRIP_W == 2 * NT16, "strip fill: two B units per thread");
  __shared__ __attribute__((aligned(16))) uint16_t As[BM16 * LROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[STRIP_W * LROW];
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask &t = tasks[e.task];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const int M = t.M, N = t.N, m0 = e.m0, n0 = e.n0;
  const int nrem = min(N - n0, STRIP_W);
  const int K = t.nseg > 0 ? t.seg[0].K : 0;   // a task without a segment stores zeros
  uint16_t *C = static_cast<uint16_t *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;

  // one operand unit of the single stage (the fields of gemm_block16's Unit)
  auto unit = [&](const DevOperand &o, bool is_a, int uidx, int first, int rem) {
    Unit u;
    const uint16_t *p = static_cast<const uint16_t *>(bases.p[o.base]) + o.off;
    const int64_t ld = o.ld;
    u.kc = is_a ? o.trans == 1 : o.trans == 0;
    u.base = u.kc ? p + (int64_t)first * ld : p + first;
    u.kstep = u.kc ? KS : (int64_t)KS * ld;
    u.ldb = (uint32_t)(ld * 2);
    const int srow = u.kc ? 4 * (uidx >> 2) : 4 * (uidx & 7), ccol = u.kc ? 8 * (uidx & 3) : 8 * (uidx >> 3);
    u.lane = (uint32_t)((int64_t)srow * ld + ccol) * 2u;
    u.s0 = srow;
    u.c0 = ccol;
    u.s_lim = u.kc ? rem : 0;
    u.c_lim = u.kc ? 0 : rem;
    return u;
  };
  if (K > 0) {
    const DevSeg &d = t.seg[0];
    u4 x[4];
    if (tid < BM16) {   // the A tile: 128 units
      const Unit u = unit(d.a, true, tid, m0, M - m0);
      load_unit(u, 0, K, x);
      store_unit<true>(As, u.kc ? tid >> 2 : tid >> 3, u.kc ? tid & 3 : tid & 7, u.kc, x);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // the B strip: 512 units
      const int uidx = tid + NT16 * h;
      const Unit u = unit(d.b, false, uidx, n0, nrem);
      load_unit(u, 0, K, x);
      store_unit<false>(Bs, u.kc ? uidx >> 2 : uidx >> 3, u.kc ? uidx & 3 : uidx & 7, u.kc, x);
    }
  }
  __syncthreads();
  u4 af[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const u4 *>(As + (64 * wm + 16 * i + r) * LROW + 8 * g);
  const int nch = (nrem + BN - 1) / BN;
  for (int ch = 0; ch < nch; ++ch) {
    f4 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f4{0, 0, 0, 0};
    if (K > 0) {
      u4 bf[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bf[j] = *reinterpret_cast<const u4 *>(Bs + (ch * BN + wn * 16 * NJ + 16 * j + r) * LROW + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = M16<H>::mma(af[i], bf[j], acc[i][j]);
    }
    // stores: lane (r, g) holds rows 64 wm + 32 h + 8 g .. +7 of each of its columns
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nl = ch * BN + wn * 16 * NJ + 16 * j + r;
      if (nl >= nrem) continue;
      const int n = n0 + nl;
      const int64_t oc = t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = m0 + 64 * wm + 32 * h + 8 * g;
        if (m >= M) continue;
        u4 y;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          y[w] = (uint32_t)from_f<H>(acc[2 * h + (w >> 1)][j][2 * (w & 1)]) |
                 ((uint32_t)from_f<H>(acc[2 * h + (w >> 1)][j][2 * (w & 1) + 1]) << 16);
        *reinterpret_cast<u4 *>(C + oc + m) = y;
      }
    }
  }
}

// ---- 256 x 256 blocks -----------------------------------------------------
//
// A 128 x 128 block moves one operand byte from L2 into LDS per 64 flops; at
// the 16-bit matrix-core rate that is more traffic than the caches deliver,
// so the final update (the launch with long K and whole output tiles) runs in
// 256 x 256 blocks instead, and so do other launches with enough such blocks
// to fill the chip (there a 128 x 128 block's 32 KB of output is too little
// to carry the fixed cost of a block).  Eight wave64s, two per SIMD, each own 128 x 64
// of the block (8 x 4 MFMA tiles: 128 accumulator registers, half of what a
// wave may hold at two waves per SIMD; one workgroup per CU).
//
// The two waves of a SIMD take turns.  Waves 0-3 (group 0) multiply while
// waves 4-7 (group 1) read their next fragments from LDS, store an operand
// stage into LDS and issue the global loads of a later one; at a barrier the
// roles swap.  One wave then keeps the SIMD's matrix pipe busy while the other
// waits on memory.  Group 0 copies the A tiles, group 1 the B tiles.  Stage s
// (32 k, counted over both K segments of the task) lives in LDS buffer s % 2:
//   phase 2s:    group 0 multiplies stage s; group 1 reads the fragments of
//                stage s, stores B(s+1), loads B(s+2)
//   phase 2s+1:  group 1 multiplies stage s; group 0 reads the fragments of
//                stage s+1, stores A(s+2), loads A(s+3)
// so stage s's buffer is read in phases 2s-1 and 2s and refilled (stage s+2)
// in phases 2s+1 and 2s+2, on the other side of a barrier.
//
// LDS rows hold 32 k (64 bytes) unpadded, the 16-byte chunk c of row L at
// position c ^ ((L >> 1) & 3): the fragment reads of 8 consecutive rows touch
// 8 distinct 16-byte bank groups.  Rows of both tiles are placed by a_lds_row,
// so a lane ends with 8 consecutive rows of C; in the B tile that only
// renames which lane owns which output column.  The loading units are laid
// out so that lanes 0-7 and 8-15 of a store instruction write rows of
// opposite parity (the other half of the banks), and every store of a unit
// sits at one of four per-thread bases plus a constant.
constexpr int BW = BW16;         // wide block rows and columns (256)
constexpr int NTW = 512;         // eight wave64s
constexpr int WROW = 32;         // LDS row stride of the wide kernel (elements)
constexpr int WTILE = BW * WROW; // elements of one operand tile of a stage

// Block column held by lane r of 16 x 16 tile j in a wave's 64 columns: the
// inverse of a_lds_row on LDS row 16 j + r.
__device__ __forceinline__ int wide_col(int j, int r) {
  return 32 * (j >> 1) + 16 * ((r >> 3) & 1) + 8 * ((r >> 2) & 1) + 4 * (j & 1) + (r & 3);
}

// One thread's share of an operand stage (256 rows of the A tile or columns of
// the B tile, 32 k), uidx = 0..255 within its group.  K-contiguous operand:
// rows 4a .. 4a+3 at k 8b .. 8b+7 (a = uidx / 4, b = uidx % 4), vector e
// holding row 4a + (e ^ (a & 1)).  Otherwise: k 4b .. 4b+3 at rows 8a .. 8a+7
// (a = uidx / 8, b = uidx % 8), vector e holding k 4b + e.
struct WSeg {
  const uint16_t *base;   // the segment's operand at (row 0 of the block, k 0)
  int64_t kstep;          // elements per stage along k
  uint32_t off0, off1;    // byte offsets of the thread's vectors 0 and 1; vectors 2, 3 lie two ld further
  uint32_t ldb2;          // two leading dimensions, in bytes
  int K;
  bool kc;
};

__device__ __forceinline__ WSeg wide_seg(const DevSeg &d, bool is_a, int uidx, int first, const Bases &bases) {
  const DevOperand &o = is_a ? d.a : d.b;
  WSeg u;
  const uint16_t *p = static_cast<const uint16_t *>(bases.p[o.base]) + o.off;
  const int64_t ld = o.ld;
  // A: trans 1 = K-contiguous; B: trans 0 = K-contiguous
  u.kc = is_a ? o.trans == 1 : o.trans == 0;
  u.base = u.kc ? p + (int64_t)first * ld : p + first;
  u.kstep = u.kc ? KS : (int64_t)KS * ld;
  u.ldb2 = (uint32_t)(ld * 4);
  // strided index of vector e: s0 + (e ^ sx); contiguous index c0
  const int s0 = u.kc ? 4 * (uidx >> 2) : 4 * (uidx & 7), sx = u.kc ? (uidx >> 2) & 1 : 0;
  const int c0 = u.kc ? 8 * (uidx & 3) : 8 * (uidx >> 3);
  u.off0 = (uint32_t)(((int64_t)(s0 + sx) * ld + c0) * 2);
  u.off1 = (uint32_t)(((int64_t)(s0 + (1 ^ sx)) * ld + c0) * 2);
  u.K = d.K;
  return u;
}

// rem: rows (A) or columns (B) of the task from the block origin
__device__ __forceinline__ void wide_load(const WSeg &u, int st, int uidx, int rem, u4 (&x)[4]) {
  const __amdgpu_buffer_rsrc_t rs = rsrc16(u.base + (int64_t)st * u.kstep);
  const int krem = u.K - st * KS;
  const int s0 = u.kc ? 4 * (uidx >> 2) : 4 * (uidx & 7), sx = u.kc ? (uidx >> 2) & 1 : 0;
  const int c0 = u.kc ? 8 * (uidx & 3) : 8 * (uidx >> 3);
  const int s_lim = u.kc ? rem : krem, c_lim = u.kc ? krem : rem;
  const bool cok = c0 < c_lim;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = cok && s0 + (e ^ sx) < s_lim;
    const uint32_t off = ((e & 1) ? u.off1 : u.off0) + (uint32_t)(e >> 1) * u.ldb2;
    x[e] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off : OOB16, 0, 0));
  }
}

// LDS stores of a unit, rows placed by a_lds_row (offsets in elements, 32
// per row).  Transposed unit (rows 8a .. 8a+7): instruction i = 4 i2 + 2 i1 + i0
// writes row m = 8a + (i ^ odd) (odd = a & 1), i.e. LDS row
//   L = 32 (a >> 2) + 16 i2 + 4 (a & 3) + 2 i1 + (i0 ^ odd),
// chunk (b >> 1) ^ i1 ^ 2 odd, half b & 1.  K-contiguous unit (rows 4a .. 4a+3):
// vector e = 2 e1 + e0 is row m = 4a + 2 e1 + (e0 ^ odd), LDS row
//   L = 32 (a >> 3) + 16 odd + 4 ((a >> 1) & 3) + 2 e1 + (e0 ^ odd),
// chunk b ^ e1 ^ 2 ((a >> 1) & 1).
__device__ __forceinline__ void wide_store(uint16_t *tile, bool kc, int uidx, const u4 (&x)[4]) {
  if (kc) {
    const int a = uidx >> 2, b = uidx & 3, odd = a & 1;
    const int base = WROW * (32 * (a >> 3) + 16 * odd + 4 * ((a >> 1) & 3));
    const int ch = b ^ (2 * ((a >> 1) & 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int e1 = e >> 1, e0 = e & 1;
      *reinterpret_cast<u4 *>(tile + base + 2 * WROW * e1 + WROW * (e0 ^ odd) + 8 * (ch ^ e1)) = x[e];
    }
  } else {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const int a = uidx >> 3, b = uidx & 7, odd = a & 1;
    const int base = WROW * (32 * (a >> 2) + 4 * (a & 3)) + 4 * (b & 1);
    const int ch = (b >> 1) ^ (2 * odd);
    // row c of the unit sits in dword c >> 1 of each vector, low half for even
    // c (selector 0x05040100), high half for odd c (0x07060302); c = i ^ odd
    const uint32_t sel_even = odd ? 0x07060302u : 0x05040100u, sel_odd = odd ? 0x05040100u : 0x07060302u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int i2 = i >> 2, i1 = (i >> 1) & 1, i0 = i & 1;
      const uint32_t sel = i0 ? sel_odd : sel_even;
      u2 y;
      y[0] = __builtin_amdgcn_perm(x[1][i >> 1], x[0][i >> 1], sel);
      y[1] = __builtin_amdgcn_perm(x[3][i >> 1], x[2][i >> 1], sel);
      *reinterpret_cast<u2 *>(tile + base + 16 * WROW * i2 + 2 * WROW * i1 + WROW * (i0 ^ odd) + 8 * (ch ^ i1)) = y;
    }
  }
}

template <typename H>
__device__ __forceinline__ void gemm_block16w(const DevTask &t, int m0, int n0, const int64_t *coltab,
                                              const Bases &bases, float alpha, float beta, float cscale) {
  // [buffer][A tile, B tile]
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2 * WTILE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                 // 0: copies A, multiplies first; 1: copies B
  const int wm = wave & 1, wn = wave >> 1;   // the wave's 128 x 64: rows 128 wm.., columns 64 wn..
  const int r = lane & 15, g = lane >> 4;
  const int M = t.M, N = t.N;

  uint16_t *C = static_cast<uint16_t *>(const_cast<void *>(bases.p[t.c_base])) + t.c_off;
  const bool fin = t.final_ != 0;
  const bool preload = fin && cscale != 0.0f;
  const bool rd = fin && beta != 0.0f && !preload;
  auto out_col = [&](int n) -> int64_t { return t.ctab < 0 ? (int64_t)n * t.ldc : coltab[t.ctab + n]; };

  // stages over both K segments
  const int K0 = t.nseg > 0 ? t.seg[0].K : 0, K1 = t.nseg > 1 ? t.seg[1].K : 0;
  const int nst0 = K0 > 0 ? (K0 + KS - 1) / KS : 0, nst1 = K1 > 0 ? (K1 + KS - 1) / KS : 0;
  const int S = nst0 + nst1;
  const int uidx = tid & 255;
  const int first = grp == 0 ? m0 : n0, rem = grp == 0 ? M - m0 : N - n0;
  WSeg u0, u1;
  if (nst0 > 0) u0 = wide_seg(t.seg[0], grp == 0, uidx, first, bases);
  if (nst1 > 0) u1 = wide_seg(t.seg[1], grp == 0, uidx, first, bases);
  // The unit's addresses are recomputed from an opaque copy of uidx at each
  // use: hoisted out of the K loop they would hold more registers than the
  // accumulators leave.
  auto fresh = [](int v) {
    asm volatile("" : "+v"(v));
    return v;
  };
  auto load = [&](int s, u4(&x)[4]) {
    if (s < nst0) wide_load(u0, s, fresh(uidx), rem, x);
    else wide_load(u1, s - nst0, fresh(uidx), rem, x);
  };
  auto store = [&](int s, const u4(&x)[4]) {
    wide_store(&lds[s & 1][grp * WTILE], s < nst0 ? u0.kc : u1.kc, fresh(uidx), x);
  };

  // the first two stages' loads go out before the C preload
  u4 x0[4], x1[4];
  if (S > 0) load(0, x0);
  if (S > 1) load(1, x1);

  f4 acc[8][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 64 * wn + wide_col(j, r);
    const int64_t oc = n < N ? out_col(n) : 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc[2 * h][j] = f4{0, 0, 0, 0};
      acc[2 * h + 1][j] = f4{0, 0, 0, 0};
      const int m = m0 + 128 * wm + 32 * h + 8 * g;
      if (preload && n < N && m < M) {
        const u4 c = *reinterpret_cast<const u4 *>(C + oc + m);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[2 * h + (e >> 2)][j][e & 3] = cscale * to_f<H>((uint16_t)(c[e >> 1] >> (16 * (e & 1))));
      }
    }
  }

  if (S > 0) {
    u4 af[8], bf[4];
    // fragment rows 128 wm + 16 i + r and 64 wn + 16 j + r: (row >> 1) & 3 is (r >> 1) & 3
    const int fa = (128 * wm + r) * WROW + 8 * (g ^ ((r >> 1) & 3));
    const int fb = WTILE + (64 * wn + r) * WROW + 8 * (g ^ ((r >> 1) & 3));
    auto read_frags = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 8; ++i) af[i] = *reinterpret_cast<const u4 *>(&lds[buf][fa + 16 * WROW * i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u4 *>(&lds[buf][fb + 16 * WROW * j]);
    };
    auto multiply = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = M16<H>::mma(af[i], bf[j], acc[i][j]);
    };
    // A phase ends at a barrier that nothing may cross: left to itself the
    // scheduler sinks MFMAs below the barrier into the memory phase, where the
    // old and new fragments are then live together.
    auto phase_end = []() {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // Global loads run two stages ahead of their LDS stores, in two register
    // sets: the memory slot of iteration t stores from set t % 2 and refills it.
    // Prologue: stage 0 and A(1) in LDS; group 0 holds A(2), A(3) in sets
    // 0, 1 and group 1 holds B(1), B(2).
    store(0, x0);
    if (grp == 0) {
      if (S > 1) store(1, x1);
      if (S > 2) load(2, x0);
      if (S > 3) load(3, x1);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x0[e] = x1[e];
      if (S > 2) load(2, x1);
    }
    // One loop for both groups, group 1 one phase ahead in barriers: iteration
    // t is (compute slot, memory slot) = phases (2t, 2t+1) for group 0 and
    // (2t-1, 2t) for group 1, whose first compute slot is the prologue's.  So
    // group 0 meets the prologue barrier before the loop and group 1 meets
    // group 0's last barrier after it: both execute 2S + 3 barriers.
    if (grp == 0) {
      phase_end();
      read_frags(0);
    }
    auto iteration = [&](int t, u4(&xs)[4]) {
      const int c = t - grp;         // stage multiplied
      if (c >= 0 && c < S) multiply();
      phase_end();
      const int q = t + 1 - grp;     // stage whose fragments are read next
      if (q < S) read_frags(q & 1);
      if (q + 1 < S) store(q + 1, xs);
      if (q + 3 < S) load(q + 3, xs);
      phase_end();
    };
    for (int t = 0; t <= S; t += 2) {
      iteration(t, x0);
      if (t + 1 <= S) iteration(t + 1, x1);
    }
    if (grp == 1) phase_end();
  }

  // epilogue: lane (r, g) holds rows 128 wm + 32 h + 8 g .. +7 of each of its columns
  // (the column offsets are computed anew rather than kept from the preload)
  const int re = fresh(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 64 * wn + wide_col(j, re);
    if (n >= N) continue;
    const int64_t oc = out_col(n);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int m = m0 + 128 * wm + 32 * h + 8 * g;
      if (m >= M) continue;
      u4 *q = reinterpret_cast<u4 *>(C + oc + m);
      u4 old = u4{0, 0, 0, 0};
      if (rd) old = *q;
      u4 z;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float v0 = acc[2 * h + (w >> 1)][j][2 * (w & 1)];
        float v1 = acc[2 * h + (w >> 1)][j][2 * (w & 1) + 1];
        if (fin) {
          v0 *= alpha;
          v1 *= alpha;
          if (rd) {
            v0 += beta * to_f<H>((uint16_t)(old[w] & 0xffffu));
            v1 += beta * to_f<H>((uint16_t)(old[w] >> 16));
          }
        }
        z[w] = (uint32_t)from_f<H>(v0) | ((uint32_t)from_f<H>(v1) << 16);
      }
      *q = z;
    }
  }
}

// STAGE only names the launch (1, 2, 3 or STAGE_SIDE), so that profiles tell
// the final update from the other wide launches.
template <typename H, int STAGE>
__global__ __launch_bounds__(NTW) void wide_gemm16_kernel(const DevTask *__restrict__ tasks,
                                                          const DevTile *__restrict__ tiles,
                                                          const int64_t *__restrict__ coltab, Bases bases,
                                                          float alpha, float beta, float cscale) {
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask &t = tasks[e.task];
  const bool fin = t.final_ != 0;
  gemm_block16w<H>(t, e.m0, e.n0, coltab, bases, fin ? alpha : 1.0f, fin ? beta : 0.0f, fin ? cscale : 0.0f);
}

template <typename H, int STAGE, int NJ>
__global__ __launch_bounds__(NT16) __attribute__((amdgpu_waves_per_eu(4)))
void grouped_gemm16_kernel(const DevTask *__restrict__ tasks, const DevTile *__restrict__ tiles,
                           const int64_t *__restrict__ coltab, Bases bases, float alpha, float beta, float cscale) {
  const DevTile e = tiles[blockIdx.x];
  if (e.task < 0) return;
  const DevTask &t = tasks[e.task];
  const bool fin = t.final_ != 0;
  gemm_block16<H, NJ>(t, e.m0, e.n0, coltab, bases, fin ? alpha : 1.0f, fin ? beta : 0.0f, fin ? cscale : 0.0f);
}

template <typename H>
__global__ void scale16_kernel(uint16_t *C, int64_t m, int64_t n, int64_t ldc, float beta) {
  const int64_t total = m * n;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = idx / m, r = idx - c * m;
    uint16_t *p = C + r + c * ldc;
    *p = beta == 0.0f ? from_f<H>(0.0f) : from_f<H>(beta * to_f<H>(*p));
  }
}

// beta/alpha for the pre-scaled C update alpha*((beta/alpha)*C + sum), used
// only when |beta/alpha| <= 1 and normal in float; otherwise 0 and the
// epilogue reads C (as in the 32/64-bit kernel).
float preload_scale16(double alpha, double beta) {
  if (beta == 0.0 || alpha == 0.0) return 0.0f;
  const double r = beta / alpha, a = r < 0 ? -r : r;
  return (a <= 1.0 && a >= 1.1754943508222875e-38) ? (float)r : 0.0f;
}

template <typename H, int NJ>
void launch16_w(int stage, dim3 grid, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                const int64_t *coltab, const Bases &bases, float a, float b, float c) {
  const dim3 block(NT16);
  if (stage == 1)
    hipLaunchKernelGGL((grouped_gemm16_kernel<H, 1, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else if (stage == 2)
    hipLaunchKernelGGL((grouped_gemm16_kernel<H, 2, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else if (stage == 3)
    hipLaunchKernelGGL((grouped_gemm16_kernel<H, 3, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a, b, c);
  else
    hipLaunchKernelGGL((grouped_gemm16_kernel<H, STAGE_SIDE, NJ>), grid, block, 0, s, tasks, tiles, coltab, bases, a,
                       b, c);
}

template <typename H>
void launch16_t(int stage, int bn, unsigned n, hipStream_t s, const DevTask *tasks, const DevTile *tiles,
                const int64_t *coltab, const Bases &bases, double alpha, double beta) {
  const float a = (float)alpha, b = (float)beta, c = preload_scale16(alpha, beta);
  if (bn == STRIP_W) {
    hipLaunchKernelGGL(strip_gemm16_kernel<H>, dim3(n), dim3(NT16), 0, s, tasks, tiles, coltab, bases);
  } else if (bn == BW) {
    if (stage == 1)
      hipLaunchKernelGGL((wide_gemm16_kernel<H, 1>), dim3(n), dim3(NTW), 0, s, tasks, tiles, coltab, bases, a, b, c);
    else if (stage == 2)
      hipLaunchKernelGGL((wide_gemm16_kernel<H, 2>), dim3(n), dim3(NTW), 0, s, tasks, tiles, coltab, bases, a, b, c);
    else if (stage == 3)
      hipLaunchKernelGGL((wide_gemm16_kernel<H, 3>), dim3(n), dim3(NTW), 0, s, tasks, tiles, coltab, bases, a, b, c);
    else
      hipLaunchKernelGGL((wide_gemm16_kernel<H, STAGE_SIDE>), dim3(n), dim3(NTW), 0, s, tasks, tiles, coltab, bases,
                         a, b, c);
  } else if (bn == Blk16<2>::BN)
    launch16_w<H, 2>(stage, dim3(n), s, tasks, tiles, coltab, bases, a, b, c);
  else
    launch16_w<H, 4>(stage, dim3(n), s, tasks, tiles, coltab, bases, a, b, c);
}

}  // namespace

int launch_grouped16(tlr_dtype dt, int stage, int bn, const DevTask *tasks, const DevTile *tiles, int64_t n_tiles,
                     const int64_t *coltab, const Bases &bases, double alpha, double beta, void *stream) {
  if (n_tiles <= 0) return 0;
  if (bn != Blk16<2>::BN && bn != Blk16<4>::BN && bn != BW && !(bn == STRIP_W && stage == 2))
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == TLR_F16)
    launch16_t<_Float16>(stage, bn, (unsigned)n_tiles, s, tasks, tiles, coltab, bases, alpha, beta);
  else
    launch16_t<__bf16>(stage, bn, (unsigned)n_tiles, s, tasks, tiles, coltab, bases, alpha, beta);
  return (int)hipGetLastError();
}

int launch_scale16(tlr_dtype dt, void *C, int64_t m, int64_t n, int64_t ldc, double beta, void *stream) {
  if (m <= 0 || n <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = m * n;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  if (dt == TLR_F16)
    hipLaunchKernelGGL(scale16_kernel<_Float16>, dim3(blocks), dim3(256), 0, s, static_cast<uint16_t *>(C), m, n,
                       ldc, (float)beta);
  else
    hipLaunchKernelGGL(scale16_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, static_cast<uint16_t *>(C), m, n, ldc,
                       (float)beta);
  return (int)hipGetLastError();
}

}  // namespace tlr
