// Kernels of the low-bit momentum state of 4-bit-Muon-GRASP ([GRASP]: notes
// on "Achieving low-bit Muon through subspace preservation and grid
// quantization", overall framework, key designs 1 and 2, full example and
// training strategy):
//
//  * the 4-bit grid code of a matrix: 128 x 128 blocks, a scale per block row
//    and per block column (largest magnitude), entries coded as
//    rint(7 x / min(row scale, column scale)) and restored as q m / 7;
//  * the 8-bit group code of the factors P (rows x k) and R (cols x k): groups
//    of 128 consecutive entries of a row, rint(127 x / scale);
//  * the momentum on the stored state, M_t = mu (M_res + P R^T) + G, rounded
//    once to fp32 (the product of the 8-bit codes is exact in the MFMA's fp32
//    accumulator: bf16 holds every code, and a group sums at most 128
//    products of at most 127^2);
//  * one warm-started power-iteration step: Q = unit columns of R_{t-1},
//    P~ = M_t Q, P = P~ U^{-1} with S = P~^T P~ = U^T U (Cholesky in fp64, the
//    QR Q factor with a positive diagonal), R = M_t^T P;
//  * the residual M_t - P R^T and its grid code.
//
// Products with fp32 operands run on the bf16 MFMA with each operand split as
// x = hi + lo (hi = bf16(x), lo = bf16(x - hi)); hi hi + hi lo + lo hi keeps
// about 16 significant bits per product, near fp32, at three MFMAs.  Code and
// scale arithmetic (decode, encode, the momentum) is fp64 on fp32 values, so
// quantisation decisions are exact: 7 x and 127 x are exact in fp64 and the
// quotient is correctly rounded before rint.
#include <float.h>

#include "muon_convert.h"
#include "muon_grasp.h"

namespace muon {

namespace {

constexpr int kGB = kGridBlock;   // grid block edge and group length (128)
constexpr int kGT = 256;          // threads per block of every kernel here

typedef __bf16 gq_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gq_f32x16 __attribute__((ext_vector_type(16)));

// NaN-propagating max / min (a NaN anywhere in a block row or column makes its
// scale NaN, and every code under that scale 0).
__device__ __forceinline__ float nan_max(float a, float b) { return (b > a || b != b) ? b : a; }
__device__ __forceinline__ float nan_min(float a, float b) { return (b < a || b != b) ? b : a; }

// rint(L x / m) in fp64 (ties to even); 0 unless 0 < m < inf.
__device__ __forceinline__ int encode(float x, float m, double levels) {
  if (!(m > 0.0f) || !(m <= FLT_MAX)) return 0;
  return static_cast<int>(rint((levels * static_cast<double>(x)) / static_cast<double>(m)));
}
// q m / L in fp64.
__device__ __forceinline__ double decode(int q, float m, double levels) {
  return (static_cast<double>(q) * static_cast<double>(m)) / levels;
}
__device__ __forceinline__ int sext4(uint32_t v) { return static_cast<int>(v << 28) >> 28; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = nan_max(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------------------
// Grid code of one 128 x 128 block (bi, bj).  Thread (wave w, lane l) holds
// rows bi*128 + w + 4 s (s < 32) and columns j = bj*128 + 2 l, j + 1; entries
// outside the matrix are 0 and are neither stored nor able to raise a scale.
// All threads of the block must call this (it synchronises once).  The
// caller has read every old scale it needs before the call.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void encode_block(const float (&x0)[32], const float (&x1)[32], float cm0, float cm1,
                                             uint8_t* codes, float* sr, float* sc, int rows, int cols, int bi,
                                             int bj, float (*cpart)[kGB]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = bj * kGB + 2 * lane;
  cpart[w][2 * lane] = cm0;
  cpart[w][2 * lane + 1] = cm1;
  __syncthreads();
  float c0 = cpart[0][2 * lane], c1 = cpart[0][2 * lane + 1];
#pragma unroll
  for (int v = 1; v < 4; ++v) {
    c0 = nan_max(c0, cpart[v][2 * lane]);
    c1 = nan_max(c1, cpart[v][2 * lane + 1]);
  }
  const int nbc = (cols + kGB - 1) / kGB;
  const int64_t cb = (cols + 1) / 2;
  if (w == 0) {
    if (j < cols) sc[static_cast<int64_t>(bi) * cols + j] = c0;
    if (j + 1 < cols) sc[static_cast<int64_t>(bi) * cols + j + 1] = c1;
  }
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const int i = bi * kGB + w + 4 * s;
    const float r = wave_max(nan_max(fabsf(x0[s]), fabsf(x1[s])));
    if (i < rows) {
      if (lane == 0) sr[static_cast<int64_t>(i) * nbc + bj] = r;
      if (j < cols) {
        const int q0 = encode(x0[s], nan_min(r, c0), 7.0);
        const int q1 = j + 1 < cols ? encode(x1[s], nan_min(r, c1), 7.0) : 0;
        codes[static_cast<int64_t>(i) * cb + (j >> 1)] = static_cast<uint8_t>((q0 & 15) | ((q1 & 15) << 4));
      }
    }
  }
}

// MODE 0: grid code of fp32 X.  MODE 1: momentum without a subspace,
// M_t = mu deq(state) + G -> fp32 (workspace and optional copy), then the new
// code of M_t in place.  MODE 2: deq(state) -> fp32 Y.
template <int MODE>
__global__ __launch_bounds__(kGT) void grid_kernel(GridArgs a) {
  __shared__ float cpart[4][kGB];
  const int b = blockIdx.z, bi = blockIdx.y, bj = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rows = a.rows, cols = a.cols;
  const int j = bj * kGB + 2 * lane;
  const bool in0 = j < cols, in1 = j + 1 < cols;
  const int nbc = (cols + kGB - 1) / kGB;
  const int64_t cb = (cols + 1) / 2;
  uint8_t* codes = static_cast<uint8_t*>(a.codes[b]);
  float* sr = static_cast<float*>(a.sr[b]);
  float* sc = static_cast<float*>(a.sc[b]);
  float oc0 = 0.0f, oc1 = 0.0f;
  if constexpr (MODE != 0) {
    if (in0) oc0 = sc[static_cast<int64_t>(bi) * cols + j];
    if (in1) oc1 = sc[static_cast<int64_t>(bi) * cols + j + 1];
  }
  float x0[32], x1[32];
  float cm0 = 0.0f, cm1 = 0.0f;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const int i = bi * kGB + w + 4 * s;
    float v0 = 0.0f, v1 = 0.0f;
    if (i < rows && in0) {
      const int64_t e = static_cast<int64_t>(i) * cols + j;
      if constexpr (MODE == 0) {
        const float* X = static_cast<const float*>(a.X[b]);
        v0 = X[e];
        if (in1) v1 = X[e + 1];
      } else {
        const float r = sr[static_cast<int64_t>(i) * nbc + bj];
        const uint32_t byte = codes[static_cast<int64_t>(i) * cb + (j >> 1)];
        const double d0 = decode(sext4(byte & 15u), nan_min(r, oc0), 7.0);
        const double d1 = in1 ? decode(sext4(byte >> 4), nan_min(r, oc1), 7.0) : 0.0;
        if constexpr (MODE == 2) {
          float* Y = static_cast<float*>(a.Y[b]);
          Y[e] = static_cast<float>(d0);
          if (in1) Y[e + 1] = static_cast<float>(d1);
        } else {
          const double g0 = load_as_f32(a.G[b], e, a.g_dtype);
          const double g1 = in1 ? static_cast<double>(load_as_f32(a.G[b], e + 1, a.g_dtype)) : 0.0;
          v0 = static_cast<float>(__dadd_rn(__dmul_rn(a.mu, d0), g0));
          v1 = in1 ? static_cast<float>(__dadd_rn(__dmul_rn(a.mu, d1), g1)) : 0.0f;
          float* mt = a.mt + static_cast<int64_t>(b) * a.s_mt;
          mt[e] = v0;
          if (in1) mt[e + 1] = v1;
          if (a.Y != nullptr) {
            float* Y = static_cast<float*>(a.Y[b]);
            Y[e] = v0;
            if (in1) Y[e + 1] = v1;
          }
        }
      }
    }
    x0[s] = v0;
    x1[s] = v1;
    cm0 = nan_max(cm0, fabsf(v0));
    cm1 = nan_max(cm1, fabsf(v1));
  }
  if constexpr (MODE != 2) encode_block(x0, x1, cm0, cm1, codes, sr, sc, rows, cols, bi, bj, cpart);
}

// ---------------------------------------------------------------------------
// 8-bit group code: one wave per (row, group of 128), lane l holding entries
// 2 l and 2 l + 1 of the group.  DEQ = 0: fp32 X -> codes, scales.  DEQ = 1:
// codes, scales -> fp32 X.
// ---------------------------------------------------------------------------
template <bool DEQ>
__global__ __launch_bounds__(kGT) void group8_kernel(Group8Args a) {
  const int b = blockIdx.z, g = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (i >= a.rows) return;  // a whole wave; nothing here synchronises
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int c = g * kGB + 2 * lane;
  const bool in0 = c < k, in1 = c + 1 < k;
  float* X = (a.Xp != nullptr ? static_cast<float*>(a.Xp[b]) : a.Xs + static_cast<int64_t>(b) * a.sX) +
             static_cast<int64_t>(i) * k;
  int8_t* q = static_cast<int8_t*>(a.codes[b]) + static_cast<int64_t>(i) * k;
  float* sp = static_cast<float*>(a.scales[b]) + static_cast<int64_t>(i) * ng + g;
  if constexpr (DEQ) {
    const float s = *sp;
    if (in0) X[c] = static_cast<float>(decode(q[c], s, 127.0));
    if (in1) X[c + 1] = static_cast<float>(decode(q[c + 1], s, 127.0));
  } else {
    const float v0 = in0 ? X[c] : 0.0f, v1 = in1 ? X[c + 1] : 0.0f;
    const float s = wave_max(nan_max(fabsf(v0), fabsf(v1)));
    if (lane == 0) *sp = s;
    if (in0) q[c] = static_cast<int8_t>(encode(v0, s, 127.0));
    if (in1) q[c + 1] = static_cast<int8_t>(encode(v1, s, 127.0));
  }
}

// ---------------------------------------------------------------------------
// Q = unit columns of deq(R_{t-1}) (n x k, fp32).  Stage 1: per chunk of 256
// rows, the fp64 sum of squares of every column.  Stage 2: every block sums
// the chunk partials in chunk order (so all blocks agree), then scales its
// rows; a zero column stays zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGT) void colsq_kernel(UnitArgs a) {
  const int b = blockIdx.y, ch = blockIdx.x;
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int8_t* q = static_cast<const int8_t*>(a.codes[b]);
  const float* sc = static_cast<const float*>(a.scales[b]);
  const int i0 = ch * kGT, i1 = min(a.n, i0 + kGT);
  for (int c = threadIdx.x; c < k; c += kGT) {
    double ss = 0.0;
    for (int i = i0; i < i1; ++i) {
      const double d = decode(q[static_cast<int64_t>(i) * k + c], sc[static_cast<int64_t>(i) * ng + c / kGB], 127.0);
      ss = fma(d, d, ss);
    }
    a.part[(static_cast<int64_t>(b) * a.nchunk + ch) * k + c] = ss;
  }
}

__global__ __launch_bounds__(kGT) void unit_columns_kernel(UnitArgs a) {
  extern __shared__ double inv[];  // k entries
  const int b = blockIdx.y, ch = blockIdx.x;
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  for (int c = threadIdx.x; c < k; c += kGT) {
    double ss = 0.0;
    for (int p = 0; p < a.nchunk; ++p) ss += a.part[(static_cast<int64_t>(b) * a.nchunk + p) * k + c];
    inv[c] = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
  }
  __syncthreads();
  const int8_t* q = static_cast<const int8_t*>(a.codes[b]);
  const float* sc = static_cast<const float*>(a.scales[b]);
  float* Q = a.Q + static_cast<int64_t>(b) * a.sQ;
  const int i0 = ch * kGT, i1 = min(a.n, i0 + kGT);
  for (int64_t e = static_cast<int64_t>(i0) * k + threadIdx.x; e < static_cast<int64_t>(i1) * k; e += kGT) {
    const int i = static_cast<int>(e / k), c = static_cast<int>(e - static_cast<int64_t>(i) * k);
    Q[e] = static_cast<float>(decode(q[e], sc[static_cast<int64_t>(i) * ng + c / kGB], 127.0) * inv[c]);
  }
}

// ---------------------------------------------------------------------------
// Tall products on the MFMA: a 128 x 128 tile of C = A B per block (4 waves,
// 64 x 64 each as 2 x 2 blocks of 32x32x16), k in stages of 32 through LDS
// with the next stage's global loads in flight during the current stage's
// MFMAs.  Operand element (row, k) sits at base + row * s_row + k * s_k with
// either k contiguous (KC) or the row index contiguous; LDS holds each
// operand as [row][k] bf16 (hi, and lo for split fp32), rows padded to 40.
// ---------------------------------------------------------------------------
constexpr int kTT = 128, kTK = 32, kTL = kTK + 8;
constexpr int kStageHalves = kTT * kTL;  // bf16 elements of one operand plane

struct TileRegs {
  float v[16];
};

// Global -> registers: the thread's four runs of 4 consecutive elements.
template <bool KC>
__device__ __forceinline__ void load_f32(const float* base, int64_t s_row, int64_t s_k, int row0, int k0, int nrows,
                                         int K, TileRegs& r) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int rr = KC ? (e >> 3) : (e & 31) * 4, kk = KC ? (e & 7) * 4 : (e >> 5);
    const int row = row0 + rr, k = k0 + kk;
    const float* src = base + static_cast<int64_t>(row) * s_row + static_cast<int64_t>(k) * s_k;
    const bool full = KC ? (row < nrows && k + 3 < K) : (row + 3 < nrows && k < K);
    if (full && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
      const float4 x = *reinterpret_cast<const float4*>(src);
      r.v[4 * p] = x.x;
      r.v[4 * p + 1] = x.y;
      r.v[4 * p + 2] = x.z;
      r.v[4 * p + 3] = x.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = KC ? (row < nrows && k + q < K) : (row + q < nrows && k < K);
        r.v[4 * p + q] = ok ? src[q] : 0.0f;
      }
    }
  }
}

// Registers -> LDS as bf16 hi (and lo = bf16(x - hi) when SPLIT).
template <bool KC, bool SPLIT>
__device__ __forceinline__ void store_split(const TileRegs& r, uint16_t* hi, uint16_t* lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int rr = KC ? (e >> 3) : (e & 31) * 4, kk = KC ? (e & 7) * 4 : (e >> 5);
    uint16_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x = r.v[4 * p + q];
      h[q] = f32_to_bf16(x);
      l[q] = SPLIT ? f32_to_bf16(x - bf16_to_f32(h[q])) : 0;
    }
    if (KC) {
      *reinterpret_cast<uint2*>(hi + rr * kTL + kk) =
          make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16));
      if (SPLIT)
        *reinterpret_cast<uint2*>(lo + rr * kTL + kk) =
            make_uint2(l[0] | (static_cast<uint32_t>(l[1]) << 16), l[2] | (static_cast<uint32_t>(l[3]) << 16));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hi[(rr + q) * kTL + kk] = h[q];
        if (SPLIT) lo[(rr + q) * kTL + kk] = l[q];
      }
    }
  }
}

// int8 codes (k contiguous) -> registers (16 per thread) -> LDS as exact bf16.
struct CodeRegs {
  int v[16];
};

__device__ __forceinline__ void load_i8(const int8_t* base, int64_t s_row, int row0, int k0, int nrows, int K,
                                        CodeRegs& r) {
  const int rr = threadIdx.x >> 1, kk = (threadIdx.x & 1) * 16;
  const int row = row0 + rr, k = k0 + kk;
  const int8_t* src = base + static_cast<int64_t>(row) * s_row + k;
  if (row < nrows && k + 15 < K && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
    const uint4 x = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 16; ++q) r.v[q] = static_cast<int8_t>((w[q >> 2] >> (8 * (q & 3))) & 0xffu);
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) r.v[q] = (row < nrows && k + q < K) ? src[q] : 0;
  }
}

__device__ __forceinline__ void store_i8(const CodeRegs& r, uint16_t* hi) {
  const int rr = threadIdx.x >> 1, kk = (threadIdx.x & 1) * 16;
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = f32x2_to_bf16x2(static_cast<float>(r.v[2 * q]), static_cast<float>(r.v[2 * q + 1]));
  *reinterpret_cast<uint4*>(hi + rr * kTL + kk) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(hi + rr * kTL + kk + 8) = make_uint4(w[4], w[5], w[6], w[7]);
}

__device__ __forceinline__ gq_f32x16 mfma(const uint4& a, const uint4& b, const gq_f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gq_bf16x8, a), __builtin_bit_cast(gq_bf16x8, b),
                                                 c, 0, 0, 0);
}

// The MFMAs of one LDS stage (two k-steps of 16) for this wave's 2 x 2 blocks.
template <bool SPLIT>
__device__ __forceinline__ void mma_stage(const uint16_t* Ah, const uint16_t* Al, const uint16_t* Bh,
                                          const uint16_t* Bl, gq_f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ar = 64 * (w >> 1) + (lane & 31), bc = 64 * (w & 1) + (lane & 31);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = 16 * s + 8 * (lane >> 5);
    uint4 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      ah[x] = *reinterpret_cast<const uint4*>(Ah + (ar + 32 * x) * kTL + k);
      bh[x] = *reinterpret_cast<const uint4*>(Bh + (bc + 32 * x) * kTL + k);
      if (SPLIT) {
        al[x] = *reinterpret_cast<const uint4*>(Al + (ar + 32 * x) * kTL + k);
        bl[x] = *reinterpret_cast<const uint4*>(Bl + (bc + 32 * x) * kTL + k);
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        acc[x][y] = mfma(ah[x], bh[y], acc[x][y]);
        if (SPLIT) {
          acc[x][y] = mfma(ah[x], bl[y], acc[x][y]);
          acc[x][y] = mfma(al[x], bh[y], acc[x][y]);
        }
      }
  }
}

__device__ __forceinline__ void zero_acc(gq_f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
}

// acc += A[row0.., kbeg..kend) B[kbeg..kend), col0..] for fp32 operands
// (split).  smem: 4 planes of kStageHalves bf16.
template <bool AKC, bool BKC>
__device__ __forceinline__ void tall_loop(const TallArgs& a, int b, int row0, int col0, int kbeg, int kend,
                                          uint16_t* smem, gq_f32x16 (&acc)[2][2]) {
  const float* A = a.A + static_cast<int64_t>(b) * a.sA;
  const float* B = a.B + static_cast<int64_t>(b) * a.sB;
  uint16_t *Ah = smem, *Al = smem + kStageHalves, *Bh = smem + 2 * kStageHalves, *Bl = smem + 3 * kStageHalves;
  TileRegs ra, rb;
  load_f32<AKC>(A, a.a_row, a.a_k, row0, kbeg, a.M, kend, ra);
  load_f32<BKC>(B, a.b_row, a.b_k, col0, kbeg, a.N, kend, rb);
  for (int k0 = kbeg; k0 < kend; k0 += kTK) {
    store_split<AKC, true>(ra, Ah, Al);
    store_split<BKC, true>(rb, Bh, Bl);
    __syncthreads();
    if (k0 + kTK < kend) {
      load_f32<AKC>(A, a.a_row, a.a_k, row0, k0 + kTK, a.M, kend, ra);
      load_f32<BKC>(B, a.b_row, a.b_k, col0, k0 + kTK, a.N, kend, rb);
    }
    mma_stage<true>(Ah, Al, Bh, Bl, acc);
    __syncthreads();
  }
}

// Tile element (row, col) of accumulator register v of block (x, y).
__device__ __forceinline__ int acc_row(int x, int v) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return 64 * (w >> 1) + 32 * x + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc_col(int y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return 64 * (w & 1) + 32 * y + (lane & 31);
}

// C (or a k-piece of C) = A B, stored fp32.  grid: (N tiles, M tiles, batch * pieces).
template <bool AKC, bool BKC>
__global__ __launch_bounds__(kGT) void tall_gemm_kernel(TallArgs a) {
  __shared__ __align__(16) uint16_t smem[4 * kStageHalves];
  const int b = blockIdx.z / a.pieces, piece = blockIdx.z - b * a.pieces;
  const int row0 = blockIdx.y * kTT, col0 = blockIdx.x * kTT;
  const int kbeg = piece * a.kchunk, kend = min(a.K, kbeg + a.kchunk);
  gq_f32x16 acc[2][2];
  zero_acc(acc);
  tall_loop<AKC, BKC>(a, b, row0, col0, kbeg, kend, smem, acc);
  float* C = a.C + static_cast<int64_t>(blockIdx.z) * a.sC;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int col = col0 + acc_col(y);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + acc_row(x, v);
        if (row < a.M && col < a.N) C[static_cast<int64_t>(row) * a.N + col] = acc[x][y][v];
      }
    }
}

// out[b] = sum over pieces p (in order) of part[b * pieces + p], count floats each.
__global__ __launch_bounds__(kGT) void sum_pieces_kernel(const float* part, int pieces, int64_t count, float* out) {
  const int b = blockIdx.y;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kGT + threadIdx.x; e < count;
       e += static_cast<int64_t>(gridDim.x) * kGT) {
    float s = 0.0f;
    for (int p = 0; p < pieces; ++p) s += part[(static_cast<int64_t>(b) * pieces + p) * count + e];
    out[static_cast<int64_t>(b) * count + e] = s;
  }
}

// ---------------------------------------------------------------------------
// M_t = mu (deq(M_res) + deq(P) deq(R)^T) + G for one 128 x 128 grid block.
// The code product runs group by group (128 k each) as exact integer sums in
// the fp32 accumulator and is scaled in fp64 by sP sR / 127^2.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGT) void recon_kernel(ReconArgs a) {
  __shared__ __align__(16) uint16_t smem[2 * kStageHalves];
  const int b = blockIdx.z, bi = blockIdx.y, bj = blockIdx.x;
  const int row0 = bi * kTT, col0 = bj * kTT;
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int8_t* Pc = static_cast<const int8_t*>(a.P_codes[b]);
  const int8_t* Rc = static_cast<const int8_t*>(a.R_codes[b]);
  const float* Ps = static_cast<const float*>(a.P_scales[b]);
  const float* Rs = static_cast<const float*>(a.R_scales[b]);
  uint16_t *Ah = smem, *Bh = smem + kStageHalves;
  double pr[2][2][16];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) pr[x][y][v] = 0.0;
  for (int g = 0; g < ng; ++g) {
    const int kbeg = g * kGB, kend = min(k, kbeg + kGB);
    gq_f32x16 acc[2][2];
    zero_acc(acc);
    CodeRegs ra, rb;
    load_i8(Pc, k, row0, kbeg, a.rows, kend, ra);
    load_i8(Rc, k, col0, kbeg, a.cols, kend, rb);
    for (int k0 = kbeg; k0 < kend; k0 += kTK) {
      store_i8(ra, Ah);
      store_i8(rb, Bh);
      __syncthreads();
      if (k0 + kTK < kend) {
        load_i8(Pc, k, row0, k0 + kTK, a.rows, kend, ra);
        load_i8(Rc, k, col0, k0 + kTK, a.cols, kend, rb);
      }
      mma_stage<false>(Ah, nullptr, Bh, nullptr, acc);
      __syncthreads();
    }
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int col = col0 + acc_col(y);
      const double sR = col < a.cols ? static_cast<double>(Rs[static_cast<int64_t>(col) * ng + g]) : 0.0;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = row0 + acc_row(x, v);
          const double sP = row < a.rows ? static_cast<double>(Ps[static_cast<int64_t>(row) * ng + g]) : 0.0;
          pr[x][y][v] += (static_cast<double>(acc[x][y][v]) * (sP * sR)) / 16129.0;
        }
    }
  }
  const uint8_t* codes = static_cast<const uint8_t*>(a.res_codes[b]);
  const float* sr = static_cast<const float*>(a.res_sr[b]);
  const float* sc = static_cast<const float*>(a.res_sc[b]);
  const int nbc = (a.cols + kGB - 1) / kGB;
  const int64_t cb = (a.cols + 1) / 2;
  float* mt = a.mt + static_cast<int64_t>(b) * a.s_mt;
  float* Y = a.Y != nullptr ? static_cast<float*>(a.Y[b]) : nullptr;
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int col = col0 + acc_col(y);
    if (col >= a.cols) continue;
    const float cs = sc[static_cast<int64_t>(bi) * a.cols + col];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + acc_row(x, v);
        if (row >= a.rows) continue;
        const int64_t e = static_cast<int64_t>(row) * a.cols + col;
        const uint32_t byte = codes[static_cast<int64_t>(row) * cb + (col >> 1)];
        const int q = sext4((col & 1) ? (byte >> 4) : (byte & 15u));
        const double res = decode(q, nan_min(sr[static_cast<int64_t>(row) * nbc + bj], cs), 7.0);
        const double g = load_as_f32(a.G[b], e, a.g_dtype);
        const float m = static_cast<float>(__dadd_rn(__dmul_rn(a.mu, __dadd_rn(res, pr[x][y][v])), g));
        mt[e] = m;
        if (Y != nullptr) Y[e] = m;
      }
  }
}

// ---------------------------------------------------------------------------
// The residual M_t - P R^T of one grid block (P R^T on the split MFMA path,
// k = the subspace rank), staged through LDS into the thread layout of
// encode_block, then its grid code.
// ---------------------------------------------------------------------------
constexpr int kRL = kTT + 1;  // staged residual row length (floats)

__global__ __launch_bounds__(kGT) void residual_kernel(ResidualArgs a) {
  __shared__ __align__(16) unsigned char raw[kTT * kRL * 4];
  static_assert(kTT * kRL * 4 >= 4 * kStageHalves * 2, "staging fits under the residual tile");
  __shared__ float cpart[4][kGB];
  uint16_t* smem = reinterpret_cast<uint16_t*>(raw);
  float* tile = reinterpret_cast<float*>(raw);
  const int b = blockIdx.z, bi = blockIdx.y, bj = blockIdx.x;
  const int row0 = bi * kTT, col0 = bj * kTT;
  gq_f32x16 acc[2][2];
  zero_acc(acc);
  tall_loop<true, true>(a.prod, b, row0, col0, 0, a.prod.K, smem, acc);
  // tall_loop ends with a barrier, so the staging area can take the tile
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) tile[acc_row(x, v) * kRL + acc_col(y)] = acc[x][y][v];
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rows = a.rows, cols = a.cols;
  const int j = col0 + 2 * lane;
  const float* mt = a.mt + static_cast<int64_t>(b) * a.s_mt;
  float x0[32], x1[32];
  float cm0 = 0.0f, cm1 = 0.0f;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const int r = w + 4 * s, i = row0 + r;
    float v0 = 0.0f, v1 = 0.0f;
    if (i < rows && j < cols) {
      const int64_t e = static_cast<int64_t>(i) * cols + j;
      v0 = mt[e] - tile[r * kRL + 2 * lane];
      if (j + 1 < cols) v1 = mt[e + 1] - tile[r * kRL + 2 * lane + 1];
    }
    x0[s] = v0;
    x1[s] = v1;
    cm0 = nan_max(cm0, fabsf(v0));
    cm1 = nan_max(cm1, fabsf(v1));
  }
  encode_block(x0, x1, cm0, cm1, static_cast<uint8_t*>(a.codes[b]), static_cast<float*>(a.sr[b]),
               static_cast<float*>(a.sc[b]), rows, cols, bi, bj, cpart);
}

// ---------------------------------------------------------------------------
// CholeskyQR.  Stage 1: fp64 partial Gram matrices S_c = P~_c^T P~_c over
// chunks of 256 rows (upper triangle, 4 x 4 register blocks, 8 rows at a
// time through LDS).  Stage 2: the partials summed in chunk order.  Stage 3
// (one block per matrix): S = U^T U by right-looking Cholesky on the upper
// triangle in fp64, then U^{-1} column by column; a pivot at or below 1e-12
// of its original diagonal (a column dependent on the earlier ones, or
// zero) gives a zero column of U^{-1}, hence of P.
// ---------------------------------------------------------------------------
constexpr int kGramRows = 8;

__global__ __launch_bounds__(kGT) void gram64_kernel(CholArgs a) {
  extern __shared__ double rowsbuf[];  // kGramRows x k
  const int b = blockIdx.y, ch = blockIdx.x;
  const int k = a.k, nb = (k + 3) / 4;
  const int npairs = nb * (nb + 1) / 2;
  const float* P = a.P + static_cast<int64_t>(b) * a.sP;
  double* out = a.spart + (static_cast<int64_t>(b) * a.nchunk + ch) * k * k;
  const int i0 = ch * kGT, i1 = min(a.m, i0 + kGT);
  for (int base = 0; base < npairs; base += 4 * kGT) {
    double acc[4][16];
    int pa[4], pb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int p = base + threadIdx.x + u * kGT;
      // pair p -> (A, B) with A <= B, row-major over the upper triangle of blocks
      int A = 0;
      int rowlen = nb;
      while (p >= rowlen && A < nb) {
        p -= rowlen;
        ++A;
        --rowlen;
      }
      pa[u] = A < nb ? A : -1;
      pb[u] = A < nb ? A + p : -1;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[u][v] = 0.0;
    }
    for (int r0 = i0; r0 < i1; r0 += kGramRows) {
      const int nr = min(kGramRows, i1 - r0);
      __syncthreads();
      for (int e = threadIdx.x; e < kGramRows * k; e += kGT) {
        const int r = e / k, c = e - r * k;
        rowsbuf[e] = r < nr ? static_cast<double>(P[static_cast<int64_t>(r0 + r) * k + c]) : 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pa[u] < 0) continue;
        for (int r = 0; r < nr; ++r) {
          const double* row = rowsbuf + r * k;
          double x[4], y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ca = 4 * pa[u] + q, cb = 4 * pb[u] + q;
            x[q] = ca < k ? row[ca] : 0.0;
            y[q] = cb < k ? row[cb] : 0.0;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int z = 0; z < 4; ++z) acc[u][4 * q + z] = fma(x[q], y[z], acc[u][4 * q + z]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (pa[u] < 0) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const int ca = 4 * pa[u] + q, cb = 4 * pb[u] + z;
          if (ca < k && cb < k && ca <= cb) out[static_cast<int64_t>(ca) * k + cb] = acc[u][4 * q + z];
        }
    }
  }
}

__global__ __launch_bounds__(kGT) void gram_sum_kernel(CholArgs a) {
  const int b = blockIdx.y;
  const int64_t kk = static_cast<int64_t>(a.k) * a.k;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kGT + threadIdx.x; e < kk;
       e += static_cast<int64_t>(gridDim.x) * kGT) {
    const int r = static_cast<int>(e / a.k), c = static_cast<int>(e - static_cast<int64_t>(r) * a.k);
    if (r > c) continue;
    double s = 0.0;
    for (int p = 0; p < a.nchunk; ++p) s += a.spart[(static_cast<int64_t>(b) * a.nchunk + p) * kk + e];
    a.S[static_cast<int64_t>(b) * kk + e] = s;
  }
}

__global__ __launch_bounds__(kGT) void chol_inv_kernel(CholArgs a) {
  extern __shared__ double lds[];  // urow[k] | diag0[k] | dead flags (as doubles)[k]
  const int b = blockIdx.x, k = a.k;
  double* U = a.S + static_cast<int64_t>(b) * k * k;  // in place: upper triangle S -> U
  double* urow = lds;
  double* diag0 = lds + k;
  double* dead = lds + 2 * k;
  for (int c = threadIdx.x; c < k; c += kGT) diag0[c] = U[static_cast<int64_t>(c) * k + c];
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    const double d = U[static_cast<int64_t>(j) * k + j];
    const bool is_dead = !(d > 1e-12 * diag0[j]) || !(diag0[j] > 0.0);
    const double piv = is_dead ? 1.0 : sqrt(d);
    for (int c = j + threadIdx.x; c < k; c += kGT) {
      const double u = c == j ? piv : (is_dead ? 0.0 : U[static_cast<int64_t>(j) * k + c] / piv);
      urow[c] = u;
      U[static_cast<int64_t>(j) * k + c] = u;
    }
    if (threadIdx.x == 0) dead[j] = is_dead ? 1.0 : 0.0;
    __syncthreads();
    if (!is_dead) {
      // S[r][c] -= U[j][r] U[j][c] for j < r <= c
      const int t = k - j - 1;
      for (int e = threadIdx.x; e < t * t; e += kGT) {
        const int r = e / t, c = e - r * t;
        if (c < r) continue;
        const int rr = j + 1 + r, cc = j + 1 + c;
        U[static_cast<int64_t>(rr) * k + cc] -= urow[rr] * urow[cc];
      }
    }
    __syncthreads();
  }
  // U^{-1} (upper): column c by one thread, bottom-up; fp32 output, zero for dead columns.
  double* V = a.Vinv64 + static_cast<int64_t>(b) * k * k;  // scratch, row-major
  float* out = a.Uinv + static_cast<int64_t>(b) * k * k;
  for (int c = threadIdx.x; c < k; c += kGT) {
    for (int i = c + 1; i < k; ++i) V[static_cast<int64_t>(i) * k + c] = 0.0;
    V[static_cast<int64_t>(c) * k + c] = 1.0 / U[static_cast<int64_t>(c) * k + c];
    for (int i = c - 1; i >= 0; --i) {
      double s = 0.0;
      for (int l = i + 1; l <= c; ++l) s = fma(U[static_cast<int64_t>(i) * k + l], V[static_cast<int64_t>(l) * k + c], s);
      V[static_cast<int64_t>(i) * k + c] = -s / U[static_cast<int64_t>(i) * k + i];
    }
    const bool zero = dead[c] != 0.0;
    for (int i = 0; i < k; ++i)
      out[static_cast<int64_t>(i) * k + c] = zero ? 0.0f : static_cast<float>(V[static_cast<int64_t>(i) * k + c]);
  }
}

__global__ void ptr_table_kernel(float* base, int64_t stride, int batch, float** out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) out[b] = base + static_cast<int64_t>(b) * stride;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static dim3 grid_blocks(int rows, int cols, int batch) {
  return dim3((cols + kGB - 1) / kGB, (rows + kGB - 1) / kGB, batch);
}

hipError_t launch_grid(const GridArgs& a, int mode, int batch, hipStream_t s) {
  const dim3 g = grid_blocks(a.rows, a.cols, batch);
  if (mode == 0) hipLaunchKernelGGL(grid_kernel<0>, g, dim3(kGT), 0, s, a);
  else if (mode == 1) hipLaunchKernelGGL(grid_kernel<1>, g, dim3(kGT), 0, s, a);
  else hipLaunchKernelGGL(grid_kernel<2>, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_group8(const Group8Args& a, bool dequantize, int batch, hipStream_t s) {
  const dim3 g((a.k + kGB - 1) / kGB, (a.rows + 3) / 4, batch);
  if (dequantize) hipLaunchKernelGGL(group8_kernel<true>, g, dim3(kGT), 0, s, a);
  else hipLaunchKernelGGL(group8_kernel<false>, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_unit_columns(const UnitArgs& a, int batch, hipStream_t s) {
  const dim3 g(a.nchunk, batch);
  hipLaunchKernelGGL(colsq_kernel, g, dim3(kGT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unit_columns_kernel, g, dim3(kGT), static_cast<size_t>(a.k) * sizeof(double), s, a);
  return hipGetLastError();
}

hipError_t launch_tall(const TallArgs& a, bool akc, bool bkc, int batch, hipStream_t s) {
  const dim3 g((a.N + kTT - 1) / kTT, (a.M + kTT - 1) / kTT, batch * a.pieces);
  if (akc && bkc) hipLaunchKernelGGL((tall_gemm_kernel<true, true>), g, dim3(kGT), 0, s, a);
  else if (akc) hipLaunchKernelGGL((tall_gemm_kernel<true, false>), g, dim3(kGT), 0, s, a);
  else if (bkc) hipLaunchKernelGGL((tall_gemm_kernel<false, true>), g, dim3(kGT), 0, s, a);
  else hipLaunchKernelGGL((tall_gemm_kernel<false, false>), g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sum_pieces(const float* part, int pieces, int64_t count, float* out, int batch, hipStream_t s) {
  int64_t blocks = (count + kGT - 1) / kGT;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(sum_pieces_kernel, dim3(static_cast<unsigned>(blocks), batch), dim3(kGT), 0, s, part, pieces,
                     count, out);
  return hipGetLastError();
}

hipError_t launch_recon(const ReconArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(recon_kernel, grid_blocks(a.rows, a.cols, batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_residual(const ResidualArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(residual_kernel, grid_blocks(a.rows, a.cols, batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cholqr(const CholArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(gram64_kernel, dim3(a.nchunk, batch), dim3(kGT),
                     static_cast<size_t>(kGramRows) * a.k * sizeof(double), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = (static_cast<int64_t>(a.k) * a.k + kGT - 1) / kGT;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gram_sum_kernel, dim3(static_cast<unsigned>(blocks), batch), dim3(kGT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chol_inv_kernel, dim3(batch), dim3(kGT), static_cast<size_t>(3) * a.k * sizeof(double), s, a);
  return hipGetLastError();
}

hipError_t launch_ptr_table(float* base, int64_t stride, int batch, float** out, hipStream_t s) {
  hipLaunchKernelGGL(ptr_table_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, base, stride, batch, out);
  return hipGetLastError();
}

}  // namespace muon
