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
// Thread layout of the grid-code kernels on block (bi, bj): thread t holds
// columns j0 = bj*128 + 8 (t % 16) .. j0 + 7 of rows bi*128 + t / 16 + 16 s
// (s < 8), so a row's 128 columns sit in 16 lanes of one wave and its codes
// are 4 bytes per thread.  `vec`: cols % 8 == 0, every 8-column run is whole
// and aligned (16-byte loads of G, 32-byte stores of M_t, 4-byte code words).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8_f32(const void* p, int64_t e, int dtype, bool vec, int n, float (&v)[8]) {
  if (vec) {
    if (dtype == 0) {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e);
      const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e + 4);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + e);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint16_t lo = static_cast<uint16_t>(w[q] & 0xffffu), hi = static_cast<uint16_t>(w[q] >> 16);
        v[2 * q] = dtype == 1 ? bf16_to_f32(lo) : f16_to_f32(lo);
        v[2 * q + 1] = dtype == 1 ? bf16_to_f32(hi) : f16_to_f32(hi);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = c < n ? load_as_f32(p, e + c, dtype) : 0.0f;
  }
}

__device__ __forceinline__ void store8_f32(float* p, bool vec, int n, const float (&v)[8]) {
  if (vec) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < n) p[c] = v[c];
  }
}

// Grid code of block (bi, bj) from the values x[s][c] of this thread (0
// outside the matrix).  All threads of the block call this; it synchronises
// once, and the caller has read every old scale it needs before the call.
__device__ __forceinline__ void encode_block(const float (&x)[8][8], uint8_t* codes, float* sr, float* sc, int rows,
                                             int cols, int bi, int bj, bool vec, float (*cpart)[kGB]) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, cg = t & 15, rs = t >> 4;
  const int j0 = bj * kGB + 8 * cg, n = min(8, cols - j0);
  const int nbc = (cols + kGB - 1) / kGB;
  const int64_t cb = (cols + 1) / 2;
  float cm[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) m = nan_max(m, fabsf(x[s][c]));
    m = nan_max(m, __shfl_xor(m, 16));
    cm[c] = nan_max(m, __shfl_xor(m, 32));
  }
  if (lane < 16)
#pragma unroll
    for (int c = 0; c < 8; ++c) cpart[w][8 * cg + c] = cm[c];
  __syncthreads();
  float cs[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    cs[c] = nan_max(nan_max(cpart[0][8 * cg + c], cpart[1][8 * cg + c]), nan_max(cpart[2][8 * cg + c], cpart[3][8 * cg + c]));
  if (t < 16)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < n) sc[static_cast<int64_t>(bi) * cols + j0 + c] = cs[c];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int i = bi * kGB + rs + 16 * s;
    float r = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) r = nan_max(r, fabsf(x[s][c]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) r = nan_max(r, __shfl_xor(r, o));
    if (i < rows && n > 0) {
      if (cg == 0) sr[static_cast<int64_t>(i) * nbc + bj] = r;
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int q = c < n ? encode(x[s][c], nan_min(r, cs[c]), 7.0) : 0;
        word |= static_cast<uint32_t>(q & 15) << (4 * c);
      }
      uint8_t* dst = codes + static_cast<int64_t>(i) * cb + (j0 >> 1);
      if (vec) {
        *reinterpret_cast<uint32_t*>(dst) = word;
      } else {
        for (int q = 0; 2 * q < n; ++q) dst[q] = static_cast<uint8_t>(word >> (8 * q));
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
  const int t = threadIdx.x, cg = t & 15, rs = t >> 4;
  const int rows = a.rows, cols = a.cols;
  const int j0 = bj * kGB + 8 * cg, n = min(8, cols - j0);
  const int nbc = (cols + kGB - 1) / kGB;
  const int64_t cb = (cols + 1) / 2;
  uint8_t* codes = static_cast<uint8_t*>(a.codes[b]);
  float* sr = static_cast<float*>(a.sr[b]);
  float* sc = static_cast<float*>(a.sc[b]);
  // vector accesses need cols % 8 == 0 and aligned bases (user pointers may be offset)
  uintptr_t mis = reinterpret_cast<uintptr_t>(codes) & 3u;
  if (MODE == 0) mis |= reinterpret_cast<uintptr_t>(a.X[b]) & 15u;
  if (MODE == 1) mis |= (reinterpret_cast<uintptr_t>(a.G[b]) | reinterpret_cast<uintptr_t>(a.mt + static_cast<int64_t>(b) * a.s_mt)) & 15u;
  if (MODE != 0 && a.Y != nullptr) mis |= reinterpret_cast<uintptr_t>(a.Y[b]) & 15u;
  const bool vec = (cols & 7) == 0 && mis == 0;
  float oc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) oc[c] = (MODE != 0 && c < n) ? sc[static_cast<int64_t>(bi) * cols + j0 + c] : 0.0f;
  float x[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int i = bi * kGB + rs + 16 * s;
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = 0.0f;
    if (i < rows && n > 0) {
      const int64_t e = static_cast<int64_t>(i) * cols + j0;
      if constexpr (MODE == 0) {
        load8_f32(a.X[b], e, 0, vec, n, v);
      } else {
        const float r = sr[static_cast<int64_t>(i) * nbc + bj];
        const uint8_t* src = codes + static_cast<int64_t>(i) * cb + (j0 >> 1);
        uint32_t word = 0;
        if (vec) {
          word = *reinterpret_cast<const uint32_t*>(src);
        } else {
          for (int q = 0; 2 * q < n; ++q) word |= static_cast<uint32_t>(src[q]) << (8 * q);
        }
        double d[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) d[c] = c < n ? decode(sext4((word >> (4 * c)) & 15u), nan_min(r, oc[c]), 7.0) : 0.0;
        if constexpr (MODE == 2) {
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = static_cast<float>(d[c]);
          store8_f32(static_cast<float*>(a.Y[b]) + e, vec, n, v);
        } else {
          float g[8];
          load8_f32(a.G[b], e, a.g_dtype, vec, n, g);
#pragma unroll
          for (int c = 0; c < 8; ++c)
            v[c] = c < n ? static_cast<float>(__dadd_rn(__dmul_rn(a.mu, d[c]), static_cast<double>(g[c]))) : 0.0f;
          store8_f32(a.mt + static_cast<int64_t>(b) * a.s_mt + e, vec, n, v);
          if (a.Y != nullptr) store8_f32(static_cast<float*>(a.Y[b]) + e, vec, n, v);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) x[s][c] = v[c];
  }
  if constexpr (MODE != 2) encode_block(x, codes, sr, sc, rows, cols, bi, bj, vec, cpart);
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
// Q = unit columns of the decoded R_{t-1} (n x k, fp32).  Stage 1: per chunk
// of kUnitRows rows, the fp64 sum of squares of every column.  Stage 2 (one
// block per matrix): 1 / norm per column from the chunk partials summed in
// chunk order (0 for a zero column).  Stage 3: the scaled rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGT) void colsq_kernel(UnitArgs a) {
  const int b = blockIdx.y, ch = blockIdx.x;
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int8_t* q = static_cast<const int8_t*>(a.codes[b]);
  const float* sc = static_cast<const float*>(a.scales[b]);
  const int i0 = ch * kUnitRows, i1 = min(a.n, i0 + kUnitRows);
  for (int c = threadIdx.x; c < k; c += kGT) {
    double ss = 0.0;
    for (int i = i0; i < i1; ++i) {
      const double d = decode(q[static_cast<int64_t>(i) * k + c], sc[static_cast<int64_t>(i) * ng + c / kGB], 127.0);
      ss = fma(d, d, ss);
    }
    a.part[(static_cast<int64_t>(b) * a.nchunk + ch) * k + c] = ss;
  }
}

__global__ __launch_bounds__(kGT) void colinv_kernel(UnitArgs a) {
  const int b = blockIdx.x, k = a.k;
  for (int c = threadIdx.x; c < k; c += kGT) {
    double ss = 0.0;
    for (int p = 0; p < a.nchunk; ++p) ss += a.part[(static_cast<int64_t>(b) * a.nchunk + p) * k + c];
    a.inv[static_cast<int64_t>(b) * k + c] = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
  }
}

__global__ __launch_bounds__(kGT) void unit_columns_kernel(UnitArgs a) {
  const int b = blockIdx.y, ch = blockIdx.x;
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int8_t* q = static_cast<const int8_t*>(a.codes[b]);
  const float* sc = static_cast<const float*>(a.scales[b]);
  const double* inv = a.inv + static_cast<int64_t>(b) * k;
  float* Q = a.Q + static_cast<int64_t>(b) * a.sQ;
  const int i0 = ch * kUnitRows, i1 = min(a.n, i0 + kUnitRows);
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
    // KC: 8 threads per row, 16 bytes each; row-contiguous: a row per thread
    // (consecutive threads on consecutive rows), 4 scalar loads along k
    const int rr = KC ? (e >> 3) : (e & 127), kk = KC ? (e & 7) * 4 : (e >> 7) * 4;
    const int row = row0 + rr, k = k0 + kk;
    const float* src = base + static_cast<int64_t>(row) * s_row + static_cast<int64_t>(k) * s_k;
    if (KC && row < nrows && k + 3 < K && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
      const float4 x = *reinterpret_cast<const float4*>(src);
      r.v[4 * p] = x.x;
      r.v[4 * p + 1] = x.y;
      r.v[4 * p + 2] = x.z;
      r.v[4 * p + 3] = x.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) r.v[4 * p + q] = (row < nrows && k + q < K) ? src[static_cast<int64_t>(q) * s_k] : 0.0f;
    }
  }
}

// Registers -> LDS as bf16 hi (and lo = bf16(x - hi) when SPLIT).
template <bool KC, bool SPLIT>
__device__ __forceinline__ void store_split(const TileRegs& r, uint16_t* hi, uint16_t* lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int rr = KC ? (e >> 3) : (e & 127), kk = KC ? (e & 7) * 4 : (e >> 7) * 4;
    uint16_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x = r.v[4 * p + q];
      h[q] = f32_to_bf16(x);
      l[q] = SPLIT ? f32_to_bf16(x - bf16_to_f32(h[q])) : 0;
    }
    *reinterpret_cast<uint2*>(hi + rr * kTL + kk) =
        make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16));
    if (SPLIT)
      *reinterpret_cast<uint2*>(lo + rr * kTL + kk) =
          make_uint2(l[0] | (static_cast<uint32_t>(l[1]) << 16), l[2] | (static_cast<uint32_t>(l[3]) << 16));
  }
}

// int8 codes (k contiguous) -> registers (16 bytes per thread, packed) -> LDS
// as exact bf16.
struct CodeRegs {
  uint4 v;
};

__device__ __forceinline__ void load_i8(const int8_t* base, int64_t s_row, int row0, int k0, int nrows, int K,
                                        CodeRegs& r) {
  const int rr = threadIdx.x >> 1, kk = (threadIdx.x & 1) * 16;
  const int row = row0 + rr, k = k0 + kk;
  const int8_t* src = base + static_cast<int64_t>(row) * s_row + k;
  if (row < nrows && k + 15 < K && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
    r.v = *reinterpret_cast<const uint4*>(src);
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (row < nrows && k + q < K) w[q >> 2] |= static_cast<uint32_t>(static_cast<uint8_t>(src[q])) << (8 * (q & 3));
    r.v = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ void store_i8(const CodeRegs& r, uint16_t* hi) {
  const int rr = threadIdx.x >> 1, kk = (threadIdx.x & 1) * 16;
  const uint32_t in[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int lo = static_cast<int8_t>((in[q >> 1] >> (16 * (q & 1))) & 0xffu);
    const int hi8 = static_cast<int8_t>((in[q >> 1] >> (16 * (q & 1) + 8)) & 0xffu);
    w[q] = f32x2_to_bf16x2(static_cast<float>(lo), static_cast<float>(hi8));
  }
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
// An operand already split into bf16 planes (hi, lo), k contiguous: the
// thread's four runs of 4 consecutive k, 8 bytes per plane each.
struct PairRegs {
  uint2 h[4], l[4];
};

__device__ __forceinline__ void load_pair(const uint16_t* hi, const uint16_t* lo, int64_t s_row, int row0, int k0,
                                          int nrows, int K, PairRegs& r) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int row = row0 + (e >> 3), k = k0 + (e & 7) * 4;
    const int64_t off = static_cast<int64_t>(row) * s_row + k;
    if (row < nrows && k + 3 < K && ((reinterpret_cast<uintptr_t>(hi + off) | reinterpret_cast<uintptr_t>(lo + off)) & 7u) == 0) {
      r.h[p] = *reinterpret_cast<const uint2*>(hi + off);
      r.l[p] = *reinterpret_cast<const uint2*>(lo + off);
    } else {
      uint32_t h[2] = {0u, 0u}, l[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row < nrows && k + q < K) {
          h[q >> 1] |= static_cast<uint32_t>(hi[off + q]) << (16 * (q & 1));
          l[q >> 1] |= static_cast<uint32_t>(lo[off + q]) << (16 * (q & 1));
        }
      r.h[p] = make_uint2(h[0], h[1]);
      r.l[p] = make_uint2(l[0], l[1]);
    }
  }
}

__device__ __forceinline__ void store_pair(const PairRegs& r, uint16_t* hi, uint16_t* lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int rr = e >> 3, kk = (e & 7) * 4;
    *reinterpret_cast<uint2*>(hi + rr * kTL + kk) = r.h[p];
    *reinterpret_cast<uint2*>(lo + rr * kTL + kk) = r.l[p];
  }
}

// acc += A B over k in [kbeg, kend).  BPS: B comes pre-split (a.Bh, a.Bl:
// planes of bf16 hi / lo, element (col, k) at col * b_row + k).
template <bool AKC, bool BKC, bool BPS = false>
__device__ __forceinline__ void tall_loop(const TallArgs& a, int b, int row0, int col0, int kbeg, int kend,
                                          uint16_t* smem, gq_f32x16 (&acc)[2][2]) {
  const float* A = a.A + static_cast<int64_t>(b) * a.sA;
  uint16_t *Ah = smem, *Al = smem + kStageHalves, *Bh = smem + 2 * kStageHalves, *Bl = smem + 3 * kStageHalves;
  TileRegs ra;
  load_f32<AKC>(A, a.a_row, a.a_k, row0, kbeg, a.M, kend, ra);
  if constexpr (BPS) {
    const uint16_t* Bhi = a.Bh + static_cast<int64_t>(b) * a.sB;
    const uint16_t* Blo = a.Bl + static_cast<int64_t>(b) * a.sB;
    PairRegs rb;
    load_pair(Bhi, Blo, a.b_row, col0, kbeg, a.N, kend, rb);
    for (int k0 = kbeg; k0 < kend; k0 += kTK) {
      store_split<AKC, true>(ra, Ah, Al);
      store_pair(rb, Bh, Bl);
      __syncthreads();
      if (k0 + kTK < kend) {
        load_f32<AKC>(A, a.a_row, a.a_k, row0, k0 + kTK, a.M, kend, ra);
        load_pair(Bhi, Blo, a.b_row, col0, k0 + kTK, a.N, kend, rb);
      }
      mma_stage<true>(Ah, Al, Bh, Bl, acc);
      __syncthreads();
    }
  } else {
    const float* B = a.B + static_cast<int64_t>(b) * a.sB;
    TileRegs rb;
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
}

// X (rows x k fp32, matrix b at X + b sX) -> planes hi, lo of X^T (k x rows,
// bf16, matrix b at + b sT): the split of an operand done once, through a
// 64 x 64 LDS tile so that both sides are coalesced.
__global__ __launch_bounds__(kGT) void split_t_kernel(const float* X, int64_t sX, int rows, int k, uint16_t* hi,
                                                      uint16_t* lo, int64_t sT) {
  __shared__ float t[64][65];
  const int b = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const float* Xm = X + static_cast<int64_t>(b) * sX;
  for (int e = threadIdx.x; e < 64 * 64; e += kGT) {
    const int r = e >> 6, c = e & 63;
    t[r][c] = (r0 + r < rows && c0 + c < k) ? Xm[static_cast<int64_t>(r0 + r) * k + c0 + c] : 0.0f;
  }
  __syncthreads();
  uint16_t* H = hi + static_cast<int64_t>(b) * sT;
  uint16_t* L = lo + static_cast<int64_t>(b) * sT;
  for (int e = threadIdx.x; e < 64 * 64; e += kGT) {
    const int c = e >> 6, r = e & 63;
    if (c0 + c < k && r0 + r < rows) {
      const float x = t[r][c];
      const uint16_t h = f32_to_bf16(x);
      H[static_cast<int64_t>(c0 + c) * rows + r0 + r] = h;
      L[static_cast<int64_t>(c0 + c) * rows + r0 + r] = f32_to_bf16(x - bf16_to_f32(h));
    }
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
template <bool AKC, bool BKC, bool BPS>
__global__ __launch_bounds__(kGT) void tall_gemm_kernel(TallArgs a) {
  __shared__ __align__(16) uint16_t smem[4 * kStageHalves];
  const int b = blockIdx.z / a.pieces, piece = blockIdx.z - b * a.pieces;
  const int row0 = blockIdx.y * kTT, col0 = blockIdx.x * kTT;
  const int kbeg = piece * a.kchunk, kend = min(a.K, kbeg + a.kchunk);
  gq_f32x16 acc[2][2];
  zero_acc(acc);
  tall_loop<AKC, BKC, BPS>(a, b, row0, col0, kbeg, kend, smem, acc);
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
// M_t = mu (deq(M_res) + deq(P) deq(R)^T) + G for a 32 x 128 tile (a quarter
// of a grid block: one 32 x 32 MFMA block per wave, so that several waves per
// SIMD hide the latency of the bandwidth-bound epilogue).  The code product runs group
// by group (128 k each) as exact integer sums in the fp32 accumulator and is
// scaled in fp64 by sP sR / 127^2; the 4-bit residual decodes in fp64.  Both
// scalings multiply by fp64 reciprocals of 7 and 127^2 (within an fp64 ulp of
// the quotients, far below the fp32 rounding of M_t).
// ---------------------------------------------------------------------------
constexpr int kRecRows = 32;

__global__ __launch_bounds__(kGT) void recon_kernel(ReconArgs a) {
  // LDS: the operand staging during the products, then the fp64 product tile
  __shared__ __align__(16) double tile[kRecRows * kTT];
  static_assert(sizeof(double) * kRecRows * kTT >= sizeof(uint16_t) * (kRecRows + kTT) * kTL, "staging fits");
  __shared__ float psc[kRecRows * (kMaxRankK / kGB)];  // P's group scales for the tile's rows
  uint16_t* smem = reinterpret_cast<uint16_t*>(tile);
  const int b = blockIdx.z, bj = blockIdx.x;
  const int row0 = blockIdx.y * kRecRows, col0 = bj * kTT, bi = row0 / kGB;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wc = 32 * w;  // wave w: the 32 x 32 block at columns wc..
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int8_t* Pc = static_cast<const int8_t*>(a.P_codes[b]);
  const int8_t* Rc = static_cast<const int8_t*>(a.R_codes[b]);
  const float* Ps = static_cast<const float*>(a.P_scales[b]);
  const float* Rs = static_cast<const float*>(a.R_scales[b]);
  uint16_t *Ah = smem, *Bh = smem + kRecRows * kTL;
  const int arows = min(a.rows, row0 + kRecRows);
  constexpr double kInvL8sq = 1.0 / 16129.0, kInv7 = 1.0 / 7.0;
  // P's scales for the tile's rows, read from LDS by the fold (the k-loop's
  // barriers order these stores before the first read)
  for (int e = threadIdx.x; e < kRecRows * ng; e += kGT) {
    const int r = e / ng;
    psc[e] = row0 + r < a.rows ? Ps[static_cast<int64_t>(row0) * ng + e] : 0.0f;
  }
  double pr[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pr[v] = 0.0;
  for (int g = 0; g < ng; ++g) {
    const int kbeg = g * kGB, kend = min(k, kbeg + kGB);
    gq_f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    CodeRegs ra, rb;
    load_i8(Pc, k, row0, kbeg, arows, kend, ra);
    load_i8(Rc, k, col0, kbeg, a.cols, kend, rb);
    for (int k0 = kbeg; k0 < kend; k0 += kTK) {
      if (threadIdx.x < 2 * kRecRows) store_i8(ra, Ah);
      store_i8(rb, Bh);
      __syncthreads();
      if (k0 + kTK < kend) {
        load_i8(Pc, k, row0, k0 + kTK, arows, kend, ra);
        load_i8(Rc, k, col0, k0 + kTK, a.cols, kend, rb);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kk = 16 * s + 8 * (lane >> 5);
        const uint4 av = *reinterpret_cast<const uint4*>(Ah + (lane & 31) * kTL + kk);
        const uint4 bv = *reinterpret_cast<const uint4*>(Bh + (wc + (lane & 31)) * kTL + kk);
        acc = mfma(av, bv, acc);
      }
      __syncthreads();
    }
    const int col = col0 + wc + (lane & 31);
    const double sR = col < a.cols ? static_cast<double>(Rs[static_cast<int64_t>(col) * ng + g]) * kInvL8sq : 0.0;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const double sP = psc[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * ng + g];
      pr[v] = fma(static_cast<double>(acc[v]), sP * sR, pr[v]);
    }
  }
  // the product tile into LDS (the last loop iteration ended with a barrier)
#pragma unroll
  for (int v = 0; v < 16; ++v) tile[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * kTT + wc + (lane & 31)] = pr[v];
  __syncthreads();
  // epilogue in the grid-code layout: thread t holds columns col0 + 8 (t % 16) .. + 7
  // of rows row0 + t / 16 + 16 s (s < 2), with vector loads and stores where aligned
  const int t = threadIdx.x, cg = t & 15, rs = t >> 4;
  const int j0 = col0 + 8 * cg, n = min(8, a.cols - j0);
  if (n <= 0) return;  // no barrier follows
  const uint8_t* codes = static_cast<const uint8_t*>(a.res_codes[b]);
  const float* sr = static_cast<const float*>(a.res_sr[b]);
  const float* sc = static_cast<const float*>(a.res_sc[b]);
  const int nbc = (a.cols + kGB - 1) / kGB;
  const int64_t cb = (a.cols + 1) / 2;
  float* mt = a.mt + static_cast<int64_t>(b) * a.s_mt;
  float* Y = a.Y != nullptr ? static_cast<float*>(a.Y[b]) : nullptr;
  uintptr_t mis = (reinterpret_cast<uintptr_t>(codes) & 3u) |
                  ((reinterpret_cast<uintptr_t>(a.G[b]) | reinterpret_cast<uintptr_t>(mt) |
                    reinterpret_cast<uintptr_t>(sc)) & 15u);
  if (Y != nullptr) mis |= reinterpret_cast<uintptr_t>(Y) & 15u;
  const bool vec = (a.cols & 7) == 0 && mis == 0;
  float cs[8];
  load8_f32(sc, static_cast<int64_t>(bi) * a.cols + j0, 0, vec, n, cs);
#pragma unroll
  for (int s = 0; s < kRecRows / 16; ++s) {
    const int r = rs + 16 * s, i = row0 + r;
    if (i >= a.rows) break;
    const float rsc = sr[static_cast<int64_t>(i) * nbc + bj];
    const uint8_t* src = codes + static_cast<int64_t>(i) * cb + (j0 >> 1);
    uint32_t word = 0;
    if (vec) {
      word = *reinterpret_cast<const uint32_t*>(src);
    } else {
      for (int q = 0; 2 * q < n; ++q) word |= static_cast<uint32_t>(src[q]) << (8 * q);
    }
    const int64_t e = static_cast<int64_t>(i) * a.cols + j0;
    float g[8], m[8];
    load8_f32(a.G[b], e, a.g_dtype, vec, n, g);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int q = sext4((word >> (4 * c)) & 15u);
      const double res = static_cast<double>(q) * static_cast<double>(nan_min(rsc, cs[c])) * kInv7;
      m[c] = static_cast<float>(fma(a.mu, res + tile[r * kTT + 8 * cg + c], static_cast<double>(g[c])));
    }
    store8_f32(mt + e, vec, n, m);
    if (Y != nullptr) store8_f32(Y + e, vec, n, m);
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
  const int t = threadIdx.x, cg = t & 15, rs = t >> 4;
  const int rows = a.rows, cols = a.cols;
  const int j0 = col0 + 8 * cg, n = min(8, cols - j0);
  const float* mt = a.mt + static_cast<int64_t>(b) * a.s_mt;
  const bool vec = (cols & 7) == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.codes[b]) & 3u) | (reinterpret_cast<uintptr_t>(mt) & 15u)) == 0;
  float x[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int r = rs + 16 * s, i = row0 + r;
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = 0.0f;
    if (i < rows && n > 0) {
      load8_f32(mt, static_cast<int64_t>(i) * cols + j0, 0, vec, n, v);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < n) v[c] -= tile[r * kRL + 8 * cg + c];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) x[s][c] = v[c];
  }
  encode_block(x, static_cast<uint8_t*>(a.codes[b]), static_cast<float*>(a.sr[b]), static_cast<float*>(a.sc[b]), rows,
               cols, bi, bj, vec, cpart);
}

// ---------------------------------------------------------------------------
// CholeskyQR: P = P~ U^{-1} with P~^T P~ = U^T U.  Stage 1: fp64 partial
// Gram matrices over chunks of 256 rows (upper triangle, 4 x 4 register
// blocks, 8 rows at a time through LDS).  Stage 2: the partials summed in
// chunk order.  Stages 3 and 4 below: the Cholesky factor and the solve.
// ---------------------------------------------------------------------------
constexpr int kGramRows = 8;

__global__ __launch_bounds__(kGT) void gram64_kernel(CholArgs a) {
  extern __shared__ double rowsbuf[];  // kGramRows x k
  const int b = blockIdx.y, ch = blockIdx.x;
  const int k = a.k, nb = (k + 3) / 4;
  const int npairs = nb * (nb + 1) / 2;
  const float* P = a.P + static_cast<int64_t>(b) * a.sP;
  double* out = a.spart + (static_cast<int64_t>(b) * a.nchunk + ch) * k * k;
  const int i0 = ch * a.chunk, i1 = min(a.m, i0 + a.chunk);
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

// Stage 3, one block per matrix: blocked right-looking Cholesky S = U^T U
// on the upper triangle (fp64, in place), panels of W <= 32 rows (W k <= 7168
// doubles, 56 KB of LDS).  Per panel: wave 0 factors the W x W diagonal block
// in registers (lane c holds column c; row j of U is broadcast lane by lane),
// all waves solve for the rest of the panel rows (U11^T U12 = S12, a column
// per thread, U11 read as LDS broadcasts), and all waves apply the panel to
// the trailing rows in global memory.  A pivot at or below 1e-12 of its
// original diagonal (or a non-positive diagonal) marks a dead column: its row
// of U becomes e_j (U_jj = 1, the rest 0), so it takes nothing from later
// columns, and the solve below zeroes its column of P.
constexpr int kPanelElems = 7168;

__device__ __forceinline__ double readlane_f64(double x, int l) {
  const int2 v = __builtin_bit_cast(int2, x);
  return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(v.x, l), __builtin_amdgcn_readlane(v.y, l)));
}

__global__ __launch_bounds__(kGT) void chol_panel_kernel(CholArgs a) {
  extern __shared__ double buf[];        // W x (k - p0) panel rows, column c - p0
  __shared__ double diag0[kMaxRankK];
  __shared__ int pdead[32];
  const int b = blockIdx.x, k = a.k, W = a.panel;
  const int lane = threadIdx.x & 63;
  double* U = a.S + static_cast<int64_t>(b) * k * k;
  int* dead = a.dead + static_cast<int64_t>(b) * k;
  for (int c = threadIdx.x; c < k; c += kGT) diag0[c] = U[static_cast<int64_t>(c) * k + c];
  __syncthreads();
  for (int p0 = 0; p0 < k; p0 += W) {
    const int pw = min(W, k - p0), wid = k - p0;
    for (int e = threadIdx.x; e < pw * wid; e += kGT) {
      const int r = e / wid, c = e - r * wid;
      buf[e] = c >= r ? U[static_cast<int64_t>(p0 + r) * k + p0 + c] : 0.0;
    }
    __syncthreads();
    // 1. the pw x pw diagonal block by wave 0 in registers: lane c holds column c
    if (threadIdx.x < 64) {
      const int c = lane;
      double d[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) d[r] = (c < pw && r <= c) ? buf[r * wid + c] : 0.0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (j < pw) {
          const double djj = readlane_f64(d[j], j);
          const bool is_dead = !(diag0[p0 + j] > 0.0) || !(djj > 1e-12 * diag0[p0 + j]);
          const double piv = is_dead ? 1.0 : sqrt(djj);
          if (c == j) d[j] = piv;
          else if (c > j) d[j] = is_dead ? 0.0 : d[j] / piv;
          if (lane == 0) pdead[j] = is_dead ? 1 : 0;
          if (!is_dead) {
#pragma unroll
            for (int r = j + 1; r < 32; ++r) {
              if (r < pw) {
                const double ujr = readlane_f64(d[j], r);
                if (c >= r) d[r] = fma(-ujr, d[j], d[r]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 32; ++r)
        if (c < pw && r <= c) buf[r * wid + c] = d[r];
    }
    __syncthreads();
    // 2. the panel rows right of the block: U11^T U12 = S12, column by column
    for (int cc = pw + threadIdx.x; cc < wid; cc += kGT) {
      double x[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) x[r] = r < pw ? buf[r * wid + cc] : 0.0;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        if (r < pw) {
          double acc = x[r];
#pragma unroll
          for (int l = 0; l < r; ++l) acc = fma(-buf[l * wid + r], x[l], acc);
          x[r] = pdead[r] ? 0.0 : acc / buf[r * wid + r];
        }
      }
#pragma unroll
      for (int r = 0; r < 32; ++r)
        if (r < pw) buf[r * wid + cc] = x[r];
    }
    if (threadIdx.x < pw) dead[p0 + threadIdx.x] = pdead[threadIdx.x];
    __syncthreads();
    for (int e = threadIdx.x; e < pw * wid; e += kGT) {
      const int r = e / wid, c = e - r * wid;
      if (c >= r) U[static_cast<int64_t>(p0 + r) * k + p0 + c] = buf[e];
    }
    // 3. trailing rows r >= p0 + pw: S[r][c] -= sum over the panel of U[j][r] U[j][c],
    // in 4 x 4 blocks (R <= C) of the trailing upper triangle
    const int t = k - p0 - pw, nb = (t + 3) / 4;
    const int npairs = nb * (nb + 1) / 2;
    for (int pidx = threadIdx.x; pidx < npairs; pidx += kGT) {
      int R = 0, rem = pidx, len = nb;
      while (rem >= len) {
        rem -= len;
        ++R;
        --len;
      }
      const int C = R + rem;
      double acc[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
      for (int jj = 0; jj < pw; ++jj) {
        const double* row = buf + jj * wid + pw;
        double x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[u] = 4 * R + u < t ? row[4 * R + u] : 0.0;
          y[u] = 4 * C + u < t ? row[4 * C + u] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = fma(x[u], y[v], acc[u][v]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * R + u, c = 4 * C + v;
          if (r < t && c < t && c >= r) U[static_cast<int64_t>(p0 + pw + r) * k + p0 + pw + c] -= acc[u][v];
        }
    }
    __syncthreads();  // the trailing rows are final before the next panel loads them
  }
}

// P = P~ U^{-1} by forward substitution along each row (P U = P~).  A block
// of 4 waves takes 4 RPW rows; column block jb (64 columns, lane l owning
// column j = 64 jb + l) first takes the finished columns of earlier blocks
// (their fp64 values in LDS times rows of U read from L2), then stages U's
// 64 x 64 diagonal block in LDS and finishes its columns one at a time, each
// broadcast from the lane that owns it.  Dead columns are zero.  fp64
// arithmetic, fp32 result.
template <int RPW>
__global__ __launch_bounds__(kGT) void row_solve_kernel(CholArgs a) {
  extern __shared__ double lds[];  // U block 64 x 64 | rows: 4 waves x RPW x k
  double* ub = lds;
  const int b = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = a.k;
  double* prow = lds + 64 * 64 + static_cast<int64_t>(w) * RPW * k;
  const double* U = a.S + static_cast<int64_t>(b) * k * k;
  const int* dead = a.dead + static_cast<int64_t>(b) * k;
  const int r0 = (blockIdx.x * 4 + w) * RPW;
  const float* Pt = a.P + static_cast<int64_t>(b) * a.sP;
  float* Po = a.Pout + static_cast<int64_t>(b) * a.sP;
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + lane, nb = min(64, k - j0);
    const bool in = j < k;
    double acc[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int r = r0 + q;
      acc[q] = in && r < a.m ? static_cast<double>(Pt[static_cast<int64_t>(r) * k + j]) : 0.0;
    }
#pragma unroll 4
    for (int l = 0; l < j0; ++l) {
      const double u = in ? U[static_cast<int64_t>(l) * k + j] : 0.0;
#pragma unroll
      for (int q = 0; q < RPW; ++q) acc[q] = fma(-prow[q * k + l], u, acc[q]);
    }
    __syncthreads();  // the previous U block is no longer read
    for (int e = threadIdx.x; e < 64 * 64; e += kGT) {
      const int rr = e >> 6, cc = e & 63;
      ub[rr * 64 + cc] = (rr < nb && cc < nb && cc >= rr) ? U[static_cast<int64_t>(j0 + rr) * k + j0 + cc] : 0.0;
    }
    __syncthreads();
    for (int q = 0; q < nb; ++q) {
      const int l = j0 + q;
      const bool dl = dead[l] != 0;
      const double diag = ub[q * 64 + q], u = ub[q * 64 + lane];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const double mine = (lane == q && !dl) ? acc[rr] / diag : 0.0;
        const double pl = __shfl(mine, q);
        if (lane > q) acc[rr] = fma(-pl, u, acc[rr]);
        if (lane == q) prow[rr * k + l] = pl;
      }
    }
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int r = r0 + q;
      if (in && r < a.m) Po[static_cast<int64_t>(r) * k + j] = static_cast<float>(prow[q * k + j]);
    }
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
  hipLaunchKernelGGL(colinv_kernel, dim3(batch), dim3(kGT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unit_columns_kernel, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tall(const TallArgs& a, bool akc, bool bkc, int batch, hipStream_t s) {
  const dim3 g((a.N + kTT - 1) / kTT, (a.M + kTT - 1) / kTT, batch * a.pieces);
  if (a.Bh != nullptr) {  // B pre-split (k contiguous)
    if (akc) hipLaunchKernelGGL((tall_gemm_kernel<true, true, true>), g, dim3(kGT), 0, s, a);
    else hipLaunchKernelGGL((tall_gemm_kernel<false, true, true>), g, dim3(kGT), 0, s, a);
  } else if (akc && bkc) {
    hipLaunchKernelGGL((tall_gemm_kernel<true, true, false>), g, dim3(kGT), 0, s, a);
  } else if (akc) {
    hipLaunchKernelGGL((tall_gemm_kernel<true, false, false>), g, dim3(kGT), 0, s, a);
  } else if (bkc) {
    hipLaunchKernelGGL((tall_gemm_kernel<false, true, false>), g, dim3(kGT), 0, s, a);
  } else {
    hipLaunchKernelGGL((tall_gemm_kernel<false, false, false>), g, dim3(kGT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_split_t(const float* X, int64_t sX, int rows, int k, uint16_t* hi, uint16_t* lo, int64_t sT,
                          int batch, hipStream_t s) {
  const dim3 g((k + 63) / 64, (rows + 63) / 64, batch);
  hipLaunchKernelGGL(split_t_kernel, g, dim3(kGT), 0, s, X, sX, rows, k, hi, lo, sT);
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
  const dim3 g((a.cols + kTT - 1) / kTT, (a.rows + kRecRows - 1) / kRecRows, batch);
  hipLaunchKernelGGL(recon_kernel, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_residual(const ResidualArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(residual_kernel, grid_blocks(a.rows, a.cols, batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gram(const CholArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(gram64_kernel, dim3(a.nchunk, batch), dim3(kGT),
                     static_cast<size_t>(kGramRows) * a.k * sizeof(double), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = (static_cast<int64_t>(a.k) * a.k + kGT - 1) / kGT;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gram_sum_kernel, dim3(static_cast<unsigned>(blocks), batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chol(const CholArgs& a, int batch, hipStream_t s) {
  CholArgs c = a;
  c.panel = 32;
  while (c.panel > 1 && c.panel * a.k > kPanelElems) c.panel >>= 1;
  hipLaunchKernelGGL(chol_panel_kernel, dim3(batch), dim3(kGT), static_cast<size_t>(c.panel) * a.k * sizeof(double), s,
                     c);
  return hipGetLastError();
}

hipError_t launch_row_solve(const CholArgs& a, int batch, hipStream_t s) {
  // rows per wave: 4 while the rows' fp64 values fit beside the U block (64 KB)
  const int rpw = a.k <= 224 ? 4 : 1;
  const size_t lds = (64 * 64 + static_cast<size_t>(4) * rpw * a.k) * sizeof(double);  // <= 64 KB
  const dim3 grid((a.m + 4 * rpw - 1) / (4 * rpw), batch);
  if (rpw == 4) hipLaunchKernelGGL(row_solve_kernel<4>, grid, dim3(kGT), lds, s, a);
  else hipLaunchKernelGGL(row_solve_kernel<1>, grid, dim3(kGT), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_ptr_table(float* base, int64_t stride, int batch, float** out, hipStream_t s) {
  hipLaunchKernelGGL(ptr_table_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, base, stride, batch, out);
  return hipGetLastError();
}

}  // namespace muon
