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
  if constexpr (MODE == 1) {
    // every load of the thread's 8 rows first, then the arithmetic and the
    // stores: the stores of M_t could alias G for the compiler, so loads
    // interleaved with them would take a memory round trip per row
    float rsc[8];
    uint32_t word[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int i = bi * kGB + rs + 16 * s;
      rsc[s] = 0.0f;
      word[s] = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) x[s][c] = 0.0f;
      if (i < rows && n > 0) {
        const int64_t e = static_cast<int64_t>(i) * cols + j0;
        rsc[s] = sr[static_cast<int64_t>(i) * nbc + bj];
        const uint8_t* src = codes + static_cast<int64_t>(i) * cb + (j0 >> 1);
        if (vec) {
          word[s] = *reinterpret_cast<const uint32_t*>(src);
        } else {
          for (int q = 0; 2 * q < n; ++q) word[s] |= static_cast<uint32_t>(src[q]) << (8 * q);
        }
        load8_f32(a.G[b], e, a.g_dtype, vec, n, x[s]);  // G, replaced by M_t below
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int i = bi * kGB + rs + 16 * s;
      if (i < rows && n > 0) {
        const int64_t e = static_cast<int64_t>(i) * cols + j0;
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const double d = c < n ? decode(sext4((word[s] >> (4 * c)) & 15u), nan_min(rsc[s], oc[c]), 7.0) : 0.0;
          v[c] = c < n ? static_cast<float>(__dadd_rn(__dmul_rn(a.mu, d), static_cast<double>(x[s][c]))) : 0.0f;
        }
        store8_f32(a.mt + static_cast<int64_t>(b) * a.s_mt + e, vec, n, v);
        if (a.Y != nullptr) store8_f32(static_cast<float*>(a.Y[b]) + e, vec, n, v);
#pragma unroll
        for (int c = 0; c < 8; ++c) x[s][c] = v[c];
      }
    }
  } else {
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
        } else {  // MODE 2: decode into Y
          const float r = sr[static_cast<int64_t>(i) * nbc + bj];
          const uint8_t* src = codes + static_cast<int64_t>(i) * cb + (j0 >> 1);
          uint32_t word = 0;
          if (vec) {
            word = *reinterpret_cast<const uint32_t*>(src);
          } else {
            for (int q = 0; 2 * q < n; ++q) word |= static_cast<uint32_t>(src[q]) << (8 * q);
          }
#pragma unroll
          for (int c = 0; c < 8; ++c)
            v[c] = c < n ? static_cast<float>(decode(sext4((word >> (4 * c)) & 15u), nan_min(r, oc[c]), 7.0)) : 0.0f;
          store8_f32(static_cast<float*>(a.Y[b]) + e, vec, n, v);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) x[s][c] = v[c];
    }
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
// Column norms of the decoded R_{t-1} (n x k).  Stage 1: per chunk of
// kUnitRows rows, the fp64 sum of squares of every column.  Stage 2 (one
// block per matrix): 1 / norm per column from the chunk partials summed in
// chunk order (0 for a zero column).  The unit columns Q themselves are never
// formed: M_t Q takes the codes and these factors (mq_kernel).
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
    // in chunk order; eight loads in flight at a time
    const double* src = a.part + static_cast<int64_t>(b) * a.nchunk * k + c;
    double ss = 0.0;
    int p = 0;
    for (; p + 8 <= a.nchunk; p += 8) {
      double x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = src[static_cast<int64_t>(p + q) * k];
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += x[q];
    }
    for (; p < a.nchunk; ++p) ss += src[static_cast<int64_t>(p) * k];
    a.inv[static_cast<int64_t>(b) * k + c] = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
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

// Registers -> LDS as bf16 hi (and lo = bf16(x - hi) when SPLIT), two
// values per conversion instruction.
template <bool KC, bool SPLIT>
__device__ __forceinline__ void store_split(const TileRegs& r, uint16_t* hi, uint16_t* lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int rr = KC ? (e >> 3) : (e & 127), kk = KC ? (e & 7) * 4 : (e >> 7) * 4;
    const float* x = &r.v[4 * p];
    const uint32_t h01 = f32x2_to_bf16x2(x[0], x[1]), h23 = f32x2_to_bf16x2(x[2], x[3]);
    *reinterpret_cast<uint2*>(hi + rr * kTL + kk) = make_uint2(h01, h23);
    if (SPLIT) {
      const uint32_t l01 = f32x2_to_bf16x2(x[0] - __uint_as_float(h01 << 16), x[1] - __uint_as_float(h01 & 0xffff0000u));
      const uint32_t l23 = f32x2_to_bf16x2(x[2] - __uint_as_float(h23 << 16), x[3] - __uint_as_float(h23 & 0xffff0000u));
      *reinterpret_cast<uint2*>(lo + rr * kTL + kk) = make_uint2(l01, l23);
    }
  }
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

// An operand already split into bf16 planes (hi, lo), k contiguous: the
// thread's four runs of 4 consecutive k, 8 bytes per plane each.
struct PairRegs {
  uint2 h[4], l[4];
};

// Addresses: the tile's first row as a uniform base, 32-bit offsets from it
// (128 rows of at most MUON_MAX_DIM entries each), so each load takes one
// address register.
__device__ __forceinline__ void load_pair(const uint16_t* hi, const uint16_t* lo, int64_t s_row, int row0, int k0,
                                          int nrows, int K, PairRegs& r) {
  const uint16_t* hb = hi + static_cast<int64_t>(row0) * s_row;
  const uint16_t* lb = lo + static_cast<int64_t>(row0) * s_row;
  const bool al = (((reinterpret_cast<uintptr_t>(hb) | reinterpret_cast<uintptr_t>(lb)) & 7u) | (s_row & 3)) == 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int row = row0 + (e >> 3), k = k0 + (e & 7) * 4;
    const uint32_t off = static_cast<uint32_t>(e >> 3) * static_cast<uint32_t>(s_row) + static_cast<uint32_t>(k);
    if (al && row < nrows && k + 3 < K) {
      r.h[p] = *reinterpret_cast<const uint2*>(hb + off);
      r.l[p] = *reinterpret_cast<const uint2*>(lb + off);
    } else {
      uint32_t h[2] = {0u, 0u}, l[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row < nrows && k + q < K) {
          h[q >> 1] |= static_cast<uint32_t>(hb[off + q]) << (16 * (q & 1));
          l[q >> 1] |= static_cast<uint32_t>(lb[off + q]) << (16 * (q & 1));
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

// acc += A B over k in [kbeg, kend) for an fp32 A that is not k-contiguous
// (M_t^T: each load instruction reads 256 contiguous bytes of a row), split as
// it is staged, and a B that comes pre-split (a.Bh, a.Bl: planes of bf16 hi /
// lo, element (col, k) at col * b_row + k).  smem holds two stages (8 planes),
// the global loads run two stages ahead of the MFMAs (two register sets) and
// a stage takes one barrier.  (The k-contiguous M_t of M_t Q, whose loads
// are 128-byte pieces of 128 rows, measured slower this way.)
__device__ __forceinline__ void tall_loop(const TallArgs& a, int b, int row0, int col0, int kbeg, int kend,
                                          uint16_t* smem, gq_f32x16 (&acc)[2][2]) {
  const float* A = a.A + static_cast<int64_t>(b) * a.sA;
  const uint16_t* Bhi = a.Bh + static_cast<int64_t>(b) * a.sB;
  const uint16_t* Blo = a.Bl + static_cast<int64_t>(b) * a.sB;
  const int nst = (kend - kbeg + kTK - 1) / kTK;
  TileRegs ra[2];
  PairRegs rb[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (q < nst) {
      load_f32<false>(A, a.a_row, a.a_k, row0, kbeg + q * kTK, a.M, kend, ra[q]);
      load_pair(Bhi, Blo, a.b_row, col0, kbeg + q * kTK, a.N, kend, rb[q]);
    }
  for (int st = 0; st < nst; st += 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (st + q < nst) {
        uint16_t* base = smem + q * 4 * kStageHalves;
        uint16_t *Ah = base, *Al = base + kStageHalves, *Bh = base + 2 * kStageHalves, *Bl = base + 3 * kStageHalves;
        store_split<false, true>(ra[q], Ah, Al);
        store_pair(rb[q], Bh, Bl);
        // LDS set q was last read two stages ago, before the previous barrier
        __syncthreads();
        const int kn = kbeg + (st + q + 2) * kTK;
        if (kn < kend) {
          load_f32<false>(A, a.a_row, a.a_k, row0, kn, a.M, kend, ra[q]);
          load_pair(Bhi, Blo, a.b_row, col0, kn, a.N, kend, rb[q]);
        }
        mma_stage<true>(Ah, Al, Bh, Bl, acc);
      }
    }
  }
  __syncthreads();  // the caller may reuse smem
}

// acc += A B over k in [kbeg, kend) with both operands pre-split into bf16
// planes, k contiguous (a.Ah / a.Al and a.Bh / a.Bl): the loads run one
// stage ahead and go to LDS unconverted.
__device__ __forceinline__ void presplit_loop(const TallArgs& a, int b, int row0, int col0, int kbeg, int kend,
                                              uint16_t* smem, gq_f32x16 (&acc)[2][2]) {
  uint16_t *Ah = smem, *Al = smem + kStageHalves, *Bh = smem + 2 * kStageHalves, *Bl = smem + 3 * kStageHalves;
  const uint16_t* Ahi = a.Ah + static_cast<int64_t>(b) * a.sA;
  const uint16_t* Alo = a.Al + static_cast<int64_t>(b) * a.sA;
  const uint16_t* Bhi = a.Bh + static_cast<int64_t>(b) * a.sB;
  const uint16_t* Blo = a.Bl + static_cast<int64_t>(b) * a.sB;
  PairRegs ra, rb;
  load_pair(Ahi, Alo, a.a_row, row0, kbeg, a.M, kend, ra);
  load_pair(Bhi, Blo, a.b_row, col0, kbeg, a.N, kend, rb);
  for (int k0 = kbeg; k0 < kend; k0 += kTK) {
    store_pair(ra, Ah, Al);
    store_pair(rb, Bh, Bl);
    __syncthreads();
    if (k0 + kTK < kend) {
      load_pair(Ahi, Alo, a.a_row, row0, k0 + kTK, a.M, kend, ra);
      load_pair(Bhi, Blo, a.b_row, col0, k0 + kTK, a.N, kend, rb);
    }
    mma_stage<true>(Ah, Al, Bh, Bl, acc);
    __syncthreads();
  }
}

// An operand exact in bf16 (codes), k contiguous: the thread's four runs of 4
// consecutive k, 8 bytes each (the hi plane of load_pair alone).
struct HiRegs {
  uint2 h[4];
};

__device__ __forceinline__ void load_hi(const uint16_t* hi, int64_t s_row, int row0, int k0, int nrows, int K,
                                        HiRegs& r) {
  const uint16_t* hb = hi + static_cast<int64_t>(row0) * s_row;
  const bool al = ((reinterpret_cast<uintptr_t>(hb) & 7u) | (s_row & 3)) == 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    const int row = row0 + (e >> 3), k = k0 + (e & 7) * 4;
    const uint32_t off = static_cast<uint32_t>(e >> 3) * static_cast<uint32_t>(s_row) + static_cast<uint32_t>(k);
    if (al && row < nrows && k + 3 < K) {
      r.h[p] = *reinterpret_cast<const uint2*>(hb + off);
    } else {
      uint32_t h[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row < nrows && k + q < K) h[q >> 1] |= static_cast<uint32_t>(hb[off + q]) << (16 * (q & 1));
      r.h[p] = make_uint2(h[0], h[1]);
    }
  }
}

__device__ __forceinline__ void store_hi(const HiRegs& r, uint16_t* hi) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = threadIdx.x + kGT * p;
    *reinterpret_cast<uint2*>(hi + (e >> 3) * kTL + (e & 7) * 4) = r.h[p];
  }
}

// The MFMAs of one LDS stage with A split (hi, lo) and B exact: two per block
// and k-step.
__device__ __forceinline__ void mma_stage_exact_b(const uint16_t* Ah, const uint16_t* Al, const uint16_t* Bh,
                                                  gq_f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ar = 64 * (w >> 1) + (lane & 31), bc = 64 * (w & 1) + (lane & 31);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = 16 * s + 8 * (lane >> 5);
    uint4 ah[2], al[2], bh[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      ah[x] = *reinterpret_cast<const uint4*>(Ah + (ar + 32 * x) * kTL + k);
      al[x] = *reinterpret_cast<const uint4*>(Al + (ar + 32 * x) * kTL + k);
      bh[x] = *reinterpret_cast<const uint4*>(Bh + (bc + 32 * x) * kTL + k);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        acc[x][y] = mfma(ah[x], bh[y], acc[x][y]);
        acc[x][y] = mfma(al[x], bh[y], acc[x][y]);
      }
  }
}

// R's codes (n x k int8, per-matrix pointers) -> bf16 (k x n), exact: the B
// operand of mq_kernel, through a 64 x 64 LDS tile so that both sides are
// coalesced.
__global__ __launch_bounds__(kGT) void codes_t_kernel(const void* const* codes, int n, int k, uint16_t* ct,
                                                      int64_t s_ct) {
  __shared__ int t[64][65];
  const int b = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int8_t* q = static_cast<const int8_t*>(codes[b]);
  int v[64 * 64 / kGT];
#pragma unroll
  for (int u = 0; u < 64 * 64 / kGT; ++u) {
    const int e = threadIdx.x + kGT * u, r = e >> 6, c = e & 63;
    const bool ok = r0 + r < n && c0 + c < k;
    v[u] = q[ok ? static_cast<int64_t>(r0 + r) * k + c0 + c : 0];
    v[u] = ok ? v[u] : 0;
  }
#pragma unroll
  for (int u = 0; u < 64 * 64 / kGT; ++u) {
    const int e = threadIdx.x + kGT * u;
    t[e >> 6][e & 63] = v[u];
  }
  __syncthreads();
  uint16_t* out = ct + static_cast<int64_t>(b) * s_ct;
#pragma unroll
  for (int u = 0; u < 64 * 64 / kGT; ++u) {
    const int e = threadIdx.x + kGT * u, c = e >> 6, r = e & 63;
    if (c0 + c < k && r0 + r < n)
      out[static_cast<int64_t>(c0 + c) * n + r0 + r] = f32_to_bf16(static_cast<float>(t[r][c]));
  }
}

// X (count fp32 per matrix, matrix b at X + b sX) -> bf16 planes hi, lo of
// the same layout (matrix b at hi + b sT, lo + b sT): the split of an operand
// done once.
__global__ __launch_bounds__(kGT) void split_kernel(const float* X, int64_t sX, int64_t count, uint16_t* hi,
                                                    uint16_t* lo, int64_t sT) {
  const int b = blockIdx.y;
  const float* Xm = X + static_cast<int64_t>(b) * sX;
  uint16_t* H = hi + static_cast<int64_t>(b) * sT;
  uint16_t* L = lo + static_cast<int64_t>(b) * sT;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kGT + threadIdx.x; e < count;
       e += static_cast<int64_t>(gridDim.x) * kGT) {
    const float x = Xm[e];
    const uint16_t h = f32_to_bf16(x);
    H[e] = h;
    L[e] = f32_to_bf16(x - bf16_to_f32(h));
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

// Tile order of the tiled state kernels (grid: x = tile column, y = tile
// row, z = matrix or matrix x k piece).  Blocks are dealt to the 8 XCDs in
// turn, each with its own L2: the linear block id is renumbered so that each
// XCD takes a contiguous run of tiles, and the run goes through groups of 8
// tile rows column by column, so the tiles in flight on one XCD share their
// operand blocks (the row blocks of the group, one column block at a time)
// through its L2 instead of fetching them again from memory.
__device__ __forceinline__ void grouped_tile(int& bi, int& bj, int& z) {
  const int64_t ncols = gridDim.x, nrows = gridDim.y;
  const int64_t G = ncols * nrows * gridDim.z;
  const int64_t p = blockIdx.x + ncols * (blockIdx.y + nrows * static_cast<int64_t>(blockIdx.z));
  const int64_t q = G >> 3, rem = G & 7, xcd = p & 7, slot = p >> 3;
  const int64_t L = xcd < rem ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
  const int64_t per = ncols * nrows;
  z = static_cast<int>(L / per);
  const int64_t t = L - z * per, g = t / (8 * ncols), w = t - g * 8 * ncols;
  const int64_t rows_in = min(static_cast<int64_t>(8), nrows - 8 * g);
  bi = static_cast<int>(8 * g + w % rows_in);
  bj = static_cast<int>(w / rows_in);
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

// P~ (or its k pieces) = M_t Q from R's codes: a 128 x 128 tile per block,
// tile column bj = 8-bit group g.  M_t's entries are scaled by s_{j,g} as they
// are staged and split; the codes (R^T, bf16) go to LDS as they are; the
// epilogue scales column c by inv_c / 127 (in fp64).  One stage of 32 k in
// flight ahead of the MFMAs; three blocks share a compute unit (30 KB of LDS,
// at most 168 registers).
static_assert(kTT == kGB, "a tile column is one 8-bit group");
__global__ __launch_bounds__(kGT, 3) void mq_kernel(MQArgs a) {
  __shared__ __align__(16) uint16_t smem[3 * kStageHalves];
  uint16_t *Ah = smem, *Al = smem + kStageHalves, *Bh = smem + 2 * kStageHalves;
  int bi, bj, z;
  grouped_tile(bi, bj, z);
  const int b = z / a.pieces, piece = z - b * a.pieces;
  const int row0 = bi * kTT, col0 = bj * kTT, g = bj;
  const int kbeg = piece * a.kchunk, kend = min(a.K, kbeg + a.kchunk);
  const int ng = (a.N + kGB - 1) / kGB;
  const float* A = a.A + static_cast<int64_t>(b) * a.sA;
  const uint16_t* Ct = a.Ct + static_cast<int64_t>(b) * a.sCt;
  const float* rs = static_cast<const float*>(a.rs[b]);
  gq_f32x16 acc[2][2];
  zero_acc(acc);
  TileRegs ra;
  HiRegs rb;
  float sv[4];
  // the thread's four k of a stage: k0 + 4 (t % 8) + q (load_f32's layout)
  auto load = [&](int k0) {
    load_f32<true>(A, a.K, 1, row0, k0, a.M, kend, ra);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = k0 + (threadIdx.x & 7) * 4 + q;
      const bool ok = j < kend;
      sv[q] = rs[ok ? static_cast<int64_t>(j) * ng + g : 0];
      sv[q] = ok ? sv[q] : 0.0f;
    }
    load_hi(Ct, a.K, col0, k0, a.N, kend, rb);
  };
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kTK) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) ra.v[4 * p + q] *= sv[q];
    store_split<true, true>(ra, Ah, Al);
    store_hi(rb, Bh);
    __syncthreads();
    if (k0 + kTK < kend) load(k0 + kTK);
    mma_stage_exact_b(Ah, Al, Bh, acc);
    __syncthreads();
  }
  const double* inv = a.inv + static_cast<int64_t>(b) * a.N;
  float* C = a.C + static_cast<int64_t>(z) * a.sC;
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int col = col0 + acc_col(y);
    const double f = col < a.N ? inv[col] * (1.0 / 127.0) : 0.0;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + acc_row(x, v);
        if (row < a.M && col < a.N)
          C[static_cast<int64_t>(row) * a.N + col] = static_cast<float>(static_cast<double>(acc[x][y][v]) * f);
      }
  }
}

// C (or a k-piece of C) = A B, stored fp32, for M_t^T P (tall_loop).  grid:
// (N tiles, M tiles, batch * pieces).
__global__ __launch_bounds__(kGT, 2) void tall_gemm_kernel(TallArgs a) {
  __shared__ __align__(16) uint16_t smem[8 * kStageHalves];
  int bi, bj, z;
  grouped_tile(bi, bj, z);
  const int b = z / a.pieces, piece = z - b * a.pieces;
  const int row0 = bi * kTT, col0 = bj * kTT;
  const int kbeg = piece * a.kchunk, kend = min(a.K, kbeg + a.kchunk);
  gq_f32x16 acc[2][2];
  zero_acc(acc);
  tall_loop(a, b, row0, col0, kbeg, kend, smem, acc);
  float* C = a.C + static_cast<int64_t>(z) * a.sC;
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
// of a grid block; wave w computes the 32 x 32 block at columns 32 w ..).
// The code product runs group by group (128 k each) on the int8 MFMA, exact
// in its int32 accumulator (a group sums at most 128 products of at most
// 127^2), and is scaled in fp64 by sP sR / 127^2; the 4-bit residual decodes
// in fp64.  Both scalings multiply by fp64 reciprocals of 7 and 127^2
// (within an fp64 ulp of the quotients, far below the fp32 rounding of M_t).
// Memory latency bounds the kernel, so a block issues the loads of two
// groups' codes and of its epilogue's operands together before it uses any
// of them: for k <= 256 one round trip to memory.
// ---------------------------------------------------------------------------
constexpr int kRecRows = 32;
constexpr int kRecLd = kGB + 16;  // LDS row of one group's codes, bytes
typedef int gq_i32x4 __attribute__((ext_vector_type(4)));
typedef int gq_i32x16 __attribute__((ext_vector_type(16)));

// One group's codes of a tile: 16 bytes of P's rows row0 + t / 8 and four of
// R's rows col0 + t / 8 + 32 p, at k = 128 g + 16 (t % 8).
struct RecCodes {
  uint4 p, r[4];
};

// 16 code bytes at base + off (base: the tile's first row, a uniform address;
// off < 2^17): one 16-byte load where the piece is whole and aligned (vec),
// else byte by byte within the row (rowin) and k < K.
__device__ __forceinline__ uint4 load_code16(const int8_t* base, uint32_t off, bool vec, bool rowin, int k, int K) {
  if (vec) return *reinterpret_cast<const uint4*>(base + off);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (rowin && k + q < K) w[q >> 2] |= static_cast<uint32_t>(static_cast<uint8_t>(base[off + q])) << (8 * (q & 3));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void load_rec_codes(const int8_t* Pc, const int8_t* Rc, int k, int row0, int col0, int rows,
                                               int cols, int g, RecCodes& c) {
  const int t = threadIdx.x, kk = g * kGB + (t & 7) * 16;
  const int8_t* pb = Pc + static_cast<int64_t>(row0) * k;
  const int8_t* rb = Rc + static_cast<int64_t>(col0) * k;
  const bool al = (((reinterpret_cast<uintptr_t>(pb) | reinterpret_cast<uintptr_t>(rb)) & 15u) | (k & 15)) == 0 &&
                  kk + 15 < k;
  const uint32_t r8 = static_cast<uint32_t>(t >> 3), uk = static_cast<uint32_t>(k);
  const bool pin = row0 + (t >> 3) < rows;
  c.p = load_code16(pb, r8 * uk + kk, al && pin, pin, kk, k);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bool rin = col0 + (t >> 3) + 32 * p < cols;
    c.r[p] = load_code16(rb, (r8 + 32 * p) * uk + kk, al && rin, rin, kk, k);
  }
}

// 8 consecutive entries of G of dtype GD (0 fp32, 1 bf16, 2 fp16) as raw
// bits (two 16-byte words for fp32, one for the 16-bit types): loaded early,
// widened where used.
template <int GD>
struct GRaw {
  uint4 w[GD == 0 ? 2 : 1];
};

template <int GD>
__device__ __forceinline__ void load8_raw(const void* p, int64_t e, bool vec, int n, GRaw<GD>& r) {
  constexpr int kWords = GD == 0 ? 8 : 4;
  uint32_t w[kWords];
  if (vec) {
    if constexpr (GD == 0) {
      r.w[0] = reinterpret_cast<const uint4*>(static_cast<const float*>(p) + e)[0];
      r.w[1] = reinterpret_cast<const uint4*>(static_cast<const float*>(p) + e)[1];
    } else {
      r.w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + e);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < kWords; ++q) w[q] = 0u;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    if (c < n) {
      if constexpr (GD == 0) w[c] = static_cast<const uint32_t*>(p)[e + c];
      else w[c >> 1] |= static_cast<uint32_t>(static_cast<const uint16_t*>(p)[e + c]) << (16 * (c & 1));
    }
#pragma unroll
  for (int q = 0; q < kWords / 4; ++q) r.w[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

template <int GD>
__device__ __forceinline__ float raw_at(const GRaw<GD>& r, int c) {
  const uint4 v = r.w[GD == 0 ? c >> 2 : 0];
  const int q = GD == 0 ? c & 3 : c >> 1;
  const uint32_t x = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
  if constexpr (GD == 0) return __uint_as_float(x);
  const uint16_t h = static_cast<uint16_t>(x >> (16 * (c & 1)));
  return GD == 1 ? bf16_to_f32(h) : f16_to_f32(h);
}

__device__ __forceinline__ void stage_rec_codes(const RecCodes& c, uint8_t* Ab, uint8_t* Bb) {
  const int t = threadIdx.x, seg = (t & 7) * 16;
  *reinterpret_cast<uint4*>(Ab + (t >> 3) * kRecLd + seg) = c.p;
#pragma unroll
  for (int p = 0; p < 4; ++p) *reinterpret_cast<uint4*>(Bb + ((t >> 3) + 32 * p) * kRecLd + seg) = c.r[p];
}

// Add group g's code product (staged in Ab, Bb), scaled, to pr.
__device__ __forceinline__ void recon_group(const uint8_t* Ab, const uint8_t* Bb, int g, int k, int ng, int col,
                                            int cols, const float* Rs, const float* psc, double (&pr)[16]) {
  const int lane = threadIdx.x & 63, wc = 32 * (threadIdx.x >> 6);
  const int steps = (min(kGB, k - g * kGB) + 31) / 32;
  gq_i32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st < steps) {
      const int kk = 32 * st + 16 * (lane >> 5);
      const gq_i32x4 av = *reinterpret_cast<const gq_i32x4*>(Ab + (lane & 31) * kRecLd + kk);
      const gq_i32x4 bv = *reinterpret_cast<const gq_i32x4*>(Bb + (wc + (lane & 31)) * kRecLd + kk);
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc, 0, 0, 0);
    }
  }
  constexpr double kInvL8sq = 1.0 / 16129.0;
  const double sR = col < cols ? static_cast<double>(Rs[static_cast<int64_t>(col) * ng + g]) * kInvL8sq : 0.0;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const double sP = psc[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * ng + g];
    pr[v] = fma(static_cast<double>(acc[v]), sP * sR, pr[v]);
  }
}

template <int GD>
__global__ __launch_bounds__(kGT, GD == 0 ? 2 : 3) void recon_kernel(ReconArgs a) {
  // LDS: two groups' codes during the product, then the fp64 product tile
  constexpr int kStage = (kRecRows + kTT) * kRecLd;
  constexpr int kLds = 2 * kStage > 8 * kRecRows * kTT ? 2 * kStage : 8 * kRecRows * kTT;
  __shared__ __align__(16) unsigned char lds[kLds];
  __shared__ float psc[kRecRows * (kMaxRankK / kGB)];  // P's group scales for the tile's rows
  static_assert(kRecRows * (kMaxRankK / kGB) <= kGT, "one scale per thread");
  double* tile = reinterpret_cast<double*>(lds);
  uint8_t* A0 = lds;
  uint8_t* B0 = A0 + kRecRows * kRecLd;
  uint8_t* A1 = lds + kStage;
  uint8_t* B1 = A1 + kRecRows * kRecLd;
  const int b = blockIdx.z, bj = blockIdx.x;
  const int row0 = blockIdx.y * kRecRows, col0 = bj * kTT, bi = row0 / kGB;
  const int t = threadIdx.x, lane = t & 63, wc = 32 * (t >> 6);
  const int k = a.k, ng = (k + kGB - 1) / kGB;
  const int8_t* Pc = static_cast<const int8_t*>(a.P_codes[b]);
  const int8_t* Rc = static_cast<const int8_t*>(a.R_codes[b]);
  const float* Ps = static_cast<const float*>(a.P_scales[b]);
  const float* Rs = static_cast<const float*>(a.R_scales[b]);
  // the first two groups' codes
  RecCodes rc0, rc1;
  load_rec_codes(Pc, Rc, k, row0, col0, a.rows, a.cols, 0, rc0);
  if (ng > 1) load_rec_codes(Pc, Rc, k, row0, col0, a.rows, a.cols, 1, rc1);
  // P's scales for the tile's rows (stored to LDS below, read after a barrier)
  const float pscale = t < kRecRows * ng && row0 + t / ng < a.rows ? Ps[static_cast<int64_t>(row0) * ng + t] : 0.0f;
  // the epilogue's operands, in the grid-code layout: thread t holds columns
  // col0 + 8 (t % 16) .. + 7 of rows row0 + t / 16 + 16 s (s < 2), with
  // vector loads and stores where aligned
  const int cg = t & 15, rs = t >> 4;
  const int j0 = col0 + 8 * cg, n = min(8, a.cols - j0);
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
  constexpr int kRecPer = kRecRows / 16;
  float cs[8], rsc[kRecPer];
  GRaw<GD> gv[kRecPer];
  uint32_t word[kRecPer];
#pragma unroll
  for (int c = 0; c < 8; ++c) cs[c] = 0.0f;
  if (n > 0) load8_f32(sc, static_cast<int64_t>(bi) * a.cols + j0, 0, vec, n, cs);
#pragma unroll
  for (int s = 0; s < kRecPer; ++s) {
    const int i = row0 + rs + 16 * s;
    rsc[s] = 0.0f;
    word[s] = 0;
    if (i < a.rows && n > 0) {
      rsc[s] = sr[static_cast<int64_t>(i) * nbc + bj];
      const uint8_t* src = codes + static_cast<int64_t>(i) * cb + (j0 >> 1);
      if (vec) {
        word[s] = *reinterpret_cast<const uint32_t*>(src);
      } else {
        for (int q = 0; 2 * q < n; ++q) word[s] |= static_cast<uint32_t>(src[q]) << (8 * q);
      }
      load8_raw<GD>(a.G[b], static_cast<int64_t>(i) * a.cols + j0, vec, n, gv[s]);
    }
  }
  psc[t] = pscale;
  double pr[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pr[v] = 0.0;
  const int col = col0 + wc + (lane & 31);
  // groups in pairs: both staged, one barrier, both products
  for (int g = 0; g < ng; g += 2) {
    if (g > 0) {
      load_rec_codes(Pc, Rc, k, row0, col0, a.rows, a.cols, g, rc0);
      if (g + 1 < ng) load_rec_codes(Pc, Rc, k, row0, col0, a.rows, a.cols, g + 1, rc1);
    }
    stage_rec_codes(rc0, A0, B0);
    if (g + 1 < ng) stage_rec_codes(rc1, A1, B1);
    __syncthreads();
    recon_group(A0, B0, g, k, ng, col, a.cols, Rs, psc, pr);
    if (g + 1 < ng) recon_group(A1, B1, g + 1, k, ng, col, a.cols, Rs, psc, pr);
    __syncthreads();
  }
  // the product tile into LDS (after the last pair's barrier)
#pragma unroll
  for (int v = 0; v < 16; ++v) tile[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * kTT + wc + (lane & 31)] = pr[v];
  __syncthreads();
  if (n <= 0) return;  // no barrier follows
  constexpr double kInv7 = 1.0 / 7.0;
#pragma unroll
  for (int s = 0; s < kRecPer; ++s) {
    const int r = rs + 16 * s, i = row0 + r;
    if (i >= a.rows) break;
    const int64_t e = static_cast<int64_t>(i) * a.cols + j0;
    float m[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int q = sext4((word[s] >> (4 * c)) & 15u);
      const double res = static_cast<double>(q) * static_cast<double>(nan_min(rsc[s], cs[c])) * kInv7;
      m[c] = static_cast<float>(fma(a.mu, res + tile[r * kTT + 8 * cg + c], static_cast<double>(raw_at<GD>(gv[s], c))));
    }
    store8_f32(mt + e, vec, n, m);
    if (Y != nullptr) store8_f32(Y + e, vec, n, m);
  }
}

// ---------------------------------------------------------------------------
// The residual M_t - P R^T of one grid block (P R^T on the split MFMA path
// from pre-split operands, k = the subspace rank), then its grid code.  The
// product tile reaches the thread layout of encode_block through LDS one half
// (64 rows) at a time, in the space of the operand staging, so a block holds
// 42 KB of LDS and, at 168 registers, three blocks share a compute unit; M_t
// is loaded after the product, its latency covered by the other blocks.
// ---------------------------------------------------------------------------
constexpr int kRL = kTT + 1;  // staged residual row length (floats)

__global__ __launch_bounds__(kGT, 3) void residual_kernel(ResidualArgs a) {
  __shared__ __align__(16) unsigned char raw[4 * kStageHalves * 2];
  static_assert(4 * kStageHalves * 2 >= (kTT / 2) * kRL * 4, "a half tile fits in the staging area");
  __shared__ float cpart[4][kGB];
  uint16_t* smem = reinterpret_cast<uint16_t*>(raw);
  float* tile = reinterpret_cast<float*>(raw);
  int bi, bj, b;
  grouped_tile(bi, bj, b);
  const int row0 = bi * kTT, col0 = bj * kTT;
  const int t = threadIdx.x, w = t >> 6, cg = t & 15, rs = t >> 4;
  const int rows = a.rows, cols = a.cols;
  const int j0 = col0 + 8 * cg, n = min(8, cols - j0);
  const float* mt = a.mt + static_cast<int64_t>(b) * a.s_mt;
  const bool vec = (cols & 7) == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.codes[b]) & 3u) | (reinterpret_cast<uintptr_t>(mt) & 15u)) == 0;
  gq_f32x16 acc[2][2];
  zero_acc(acc);
  presplit_loop(a.prod, b, row0, col0, 0, a.prod.K, smem, acc);
  // this thread's M_t values (rows row0 + t / 16 + 16 s)
  float x[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int i = row0 + rs + 16 * s;
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = 0.0f;
    if (i < rows && n > 0) load8_f32(mt, static_cast<int64_t>(i) * cols + j0, 0, vec, n, v);
#pragma unroll
    for (int c = 0; c < 8; ++c) x[s][c] = v[c];
  }
  // the product, half h (rows 64 h ..) from waves 2 h and 2 h + 1; the loop
  // ended with a barrier, so the staging area can take it
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if ((w >> 1) == h)
#pragma unroll
      for (int xx = 0; xx < 2; ++xx)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int v = 0; v < 16; ++v) tile[(acc_row(xx, v) - 64 * h) * kRL + acc_col(y)] = acc[xx][y][v];
    __syncthreads();
#pragma unroll
    for (int s = 4 * h; s < 4 * h + 4; ++s) {
      const int r = rs + 16 * s, i = row0 + r;
      if (i < rows)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c < n) x[s][c] -= tile[(r - 64 * h) * kRL + 8 * cg + c];
    }
    __syncthreads();
  }
  encode_block(x, static_cast<uint8_t*>(a.codes[b]), static_cast<float*>(a.sr[b]), static_cast<float*>(a.sc[b]), rows,
               cols, bi, bj, vec, cpart);
}

// ---------------------------------------------------------------------------
// CholeskyQR: P = P~ U^{-1} with P~^T P~ = U^T U.  Stage 1: fp64 partial
// Gram matrices over row chunks of gram_chunk_rows rows (here for k > 256:
// upper triangle, 4 x 4 register blocks, 8 rows at a time through LDS; the
// fp64 MFMA kernel below for smaller k).  Stage 2: the partials summed in
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

// Stage 1 for k <= kRegRankK on the fp64 MFMA.  Block (chunk, pass, matrix)
// adds, over the chunk's rows, p_r p_r^T into the 16 x 16 blocks (I, J),
// I <= J, of the upper triangle, numbered row by row; the pass takes 32 of
// them, 8 per wave, each in one accumulator (v_mfma_f64_16x16x4f64, 4 rows
// per instruction: lane l gives A[l % 16][l / 16] = P~[r + l / 16][16 I +
// l % 16] and B[l / 16][l % 16] = P~[r + l / 16][16 J + l % 16], and holds
// D[l / 16 + 4 v][l % 16] in register v).  Rows come through LDS 64 at a
// time as fp32 (exact in fp64), zero past the chunk and past column k.
constexpr int kGramMfmaRows = 64;
constexpr int kGramMfmaLd = kRegRankK + 16;  // row stride: consecutive rows 16 banks apart
constexpr int kGramPairsPerWave = 8;
constexpr int kGramPairsPerPass = 4 * kGramPairsPerWave;
typedef double gq_f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kGT) void gram_mfma_kernel(CholArgs a) {
  __shared__ __align__(16) float rows[kGramMfmaRows * kGramMfmaLd];
  const int ch = blockIdx.x, pass = blockIdx.y, b = blockIdx.z;
  const int k = a.k, nbk = (k + 15) / 16, kw = 16 * nbk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* P = a.P + static_cast<int64_t>(b) * a.sP;
  const int i0 = ch * a.chunk, i1 = min(a.m, i0 + a.chunk);
  int pI[kGramPairsPerWave], pJ[kGramPairsPerWave];
  gq_f64x4 acc[kGramPairsPerWave];
#pragma unroll
  for (int q = 0; q < kGramPairsPerWave; ++q) {
    int p = pass * kGramPairsPerPass + w * kGramPairsPerWave + q, I = 0, len = nbk;
    while (p >= len && I < nbk) {
      p -= len;
      ++I;
      --len;
    }
    pI[q] = I < nbk ? I : -1;
    pJ[q] = I < nbk ? I + p : -1;
    acc[q] = gq_f64x4{0.0, 0.0, 0.0, 0.0};
  }
  // rows staged 4 floats per thread and load, every load of a chunk in flight at once
  const int kw4 = kw / 4;
  const bool vec = (k & 3) == 0 && (reinterpret_cast<uintptr_t>(P) & 15u) == 0;
  for (int r0 = i0; r0 < i1; r0 += kGramMfmaRows) {
    const int nr = min(kGramMfmaRows, i1 - r0);
    __syncthreads();  // the previous rows are no longer read
    float4 v[kGramMfmaRows * (kRegRankK / 4) / kGT];
#pragma unroll
    for (int q = 0; q < kGramMfmaRows * (kRegRankK / 4) / kGT; ++q) {
      const int e = threadIdx.x + q * kGT, rr = e / kw4, c = 4 * (e - rr * kw4);
      v[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (e < kGramMfmaRows * kw4 && rr < nr) {
        const float* src = P + static_cast<int64_t>(r0 + rr) * k + c;
        if (vec) {
          if (c < k) v[q] = *reinterpret_cast<const float4*>(src);  // k % 4 == 0: whole or outside
        } else {
          v[q].x = c < k ? src[0] : 0.0f;
          v[q].y = c + 1 < k ? src[1] : 0.0f;
          v[q].z = c + 2 < k ? src[2] : 0.0f;
          v[q].w = c + 3 < k ? src[3] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kGramMfmaRows * (kRegRankK / 4) / kGT; ++q) {
      const int e = threadIdx.x + q * kGT, rr = e / kw4, c = 4 * (e - rr * kw4);
      if (e < kGramMfmaRows * kw4) *reinterpret_cast<float4*>(rows + rr * kGramMfmaLd + c) = v[q];
    }
    __syncthreads();
    for (int s0 = 0; s0 < nr; s0 += 4) {
      const float* row = rows + (s0 + (lane >> 4)) * kGramMfmaLd + (lane & 15);
#pragma unroll
      for (int q = 0; q < kGramPairsPerWave; ++q)
        if (pI[q] >= 0)
          acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(row[16 * pI[q]]),
                                                        static_cast<double>(row[16 * pJ[q]]), acc[q], 0, 0, 0);
    }
  }
  double* out = a.spart + (static_cast<int64_t>(b) * a.nchunk + ch) * k * k;
#pragma unroll
  for (int q = 0; q < kGramPairsPerWave; ++q)
    if (pI[q] >= 0)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * pI[q] + (lane >> 4) + 4 * v, j = 16 * pJ[q] + (lane & 15);
        if (i < k && j < k) out[static_cast<int64_t>(i) * k + j] = acc[q][v];
      }
}

__global__ __launch_bounds__(kGT) void gram_sum_kernel(CholArgs a) {
  const int b = blockIdx.y;
  const int64_t kk = static_cast<int64_t>(a.k) * a.k;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kGT + threadIdx.x; e < kk;
       e += static_cast<int64_t>(gridDim.x) * kGT) {
    const int r = static_cast<int>(e / a.k), c = static_cast<int>(e - static_cast<int64_t>(r) * a.k);
    if (r > c) continue;
    // in chunk order; eight loads in flight at a time
    const double* src = a.spart + static_cast<int64_t>(b) * a.nchunk * kk + e;
    double s = 0.0;
    int p = 0;
    for (; p + 8 <= a.nchunk; p += 8) {
      double x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = src[static_cast<int64_t>(p + q) * kk];
#pragma unroll
      for (int q = 0; q < 8; ++q) s += x[q];
    }
    for (; p < a.nchunk; ++p) s += src[static_cast<int64_t>(p) * kk];
    a.S[static_cast<int64_t>(b) * kk + e] = s;
  }
}

// Stage 3 for k > 256 (the register-resident kernel below takes smaller k),
// one block per matrix: blocked right-looking Cholesky S = U^T U on the
// upper triangle (fp64, in place), panels of W <= 32 rows (W k <= 7168
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

// P = P~ U^{-1} as a blocked solve on the fp64 MFMA (P U = P~, column
// blocks of 64).  First U's 64 x 64 diagonal blocks are inverted (Dinv, with
// the columns of dead rows zero, so dead columns of P are zero as in the
// substitution: a dead row of U is e_p and feeds no later column).  Then a
// wave takes 16 rows and, block by block, forms A = P~[:, blk] - X[:, :j0]
// U[:j0, blk] and X[:, blk] = A Dinv_blk; its X rows stay in LDS as the A
// operand of later blocks.  fp64 arithmetic, fp32 result.
typedef double gq_f64x4 __attribute__((ext_vector_type(4)));
constexpr int kSolveBlk = 64;

// Row r (lane r) of Dinv_jb by substitution: x = e_r, then for c = 0..nb-1
// x_c *= 1 / U_cc (zero for a dead c) and x_c' -= x_c U_cc' for c' > c.  The
// block is staged in LDS first (a row per load instruction across the lanes)
// and the reciprocals are formed in parallel, so the chain from one c to the
// next is a multiply and an FMA.  Rows and columns past the matrix come out
// zero.
__global__ __launch_bounds__(kSolveBlk) void diag_inv_kernel(CholArgs a) {
  __shared__ double ub[kSolveBlk * kSolveBlk];
  __shared__ double rdg[kSolveBlk];
  const int jb = blockIdx.x, b = blockIdx.y, r = threadIdx.x;
  const int k = a.k, j0 = jb * kSolveBlk, nb = min(kSolveBlk, k - j0), nbk = (k + kSolveBlk - 1) / kSolveBlk;
  const double* U = a.S + static_cast<int64_t>(b) * k * k + static_cast<int64_t>(j0) * k + j0;
  {
    double v[kSolveBlk];
#pragma unroll
    for (int c = 0; c < kSolveBlk; ++c) {
      const bool ok = c < nb && r < nb;
      v[c] = U[ok ? static_cast<int64_t>(c) * k + r : 0];
      v[c] = ok ? v[c] : 0.0;
    }
    const bool live = r < nb && a.dead[static_cast<int64_t>(b) * k + j0 + (r < nb ? r : 0)] == 0;
    const double d = U[r < nb ? static_cast<int64_t>(r) * k + r : 0];
#pragma unroll
    for (int c = 0; c < kSolveBlk; ++c) ub[c * kSolveBlk + r] = v[c];
    rdg[r] = live ? 1.0 / d : 0.0;
  }
  __syncthreads();
  double x[kSolveBlk];
#pragma unroll
  for (int c = 0; c < kSolveBlk; ++c) x[c] = c == r ? 1.0 : 0.0;
#pragma unroll
  for (int c = 0; c < kSolveBlk; ++c) {
    x[c] *= rdg[c];
#pragma unroll
    for (int c2 = c + 1; c2 < kSolveBlk; ++c2) x[c2] = fma(-x[c], ub[c * kSolveBlk + c2], x[c2]);
  }
  double* out = a.dinv + ((static_cast<int64_t>(b) * nbk + jb) * kSolveBlk + r) * kSolveBlk;
#pragma unroll
  for (int c = 0; c < kSolveBlk; ++c) out[c] = x[c];
}

__global__ __launch_bounds__(64) void row_solve_mfma_kernel(CholArgs a) {
  extern __shared__ double xs[];  // this wave's 16 rows of X, row length ld
  const int b = blockIdx.y, lane = threadIdx.x;
  const int k = a.k, nbk = (k + kSolveBlk - 1) / kSolveBlk, ld = kSolveBlk * nbk + 1;
  const int r0 = blockIdx.x * 16;
  const int dr = lane >> 4, dc = lane & 15;  // D and B layouts: row (or k) dr (+ 4 v), column dc
  const int ar = lane & 15, ak = lane >> 4;  // A layout: row ar, k ak
  const float* Pt = a.P + static_cast<int64_t>(b) * a.sP;
  float* Po = a.Pout + static_cast<int64_t>(b) * a.sP;
  const double* U = a.S + static_cast<int64_t>(b) * k * k;
  const double* Dv = a.dinv + static_cast<int64_t>(b) * nbk * kSolveBlk * kSolveBlk;
  for (int jb = 0; jb < nbk; ++jb) {
    const int j0 = jb * kSolveBlk;
    // P~'s block: every load issued (from a clamped address) before any is used
    float pv[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + dr + 4 * v, col = j0 + 16 * t + dc;
        const bool ok = row < a.m && col < k;
        pv[t][v] = Pt[ok ? static_cast<int64_t>(row) * k + col : 0];
        pv[t][v] = ok ? pv[t][v] : 0.0f;
      }
    gq_f64x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[t][v] = static_cast<double>(pv[t][v]);
    // A = P~[:, blk] - X[:, :j0] U[:j0, blk], four k-steps per trip.  U's
    // entries for the next trip are loaded before this trip's MFMAs; loads
    // and MFMAs are unconditional (entries outside U[:j0, :k] read as zero
    // from a clamped address), so nothing branches around them.
    double bn[4][4];
    auto load_u = [&](int s0, double (&bv)[4][4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = s0 + 4 * q + dr, col = j0 + 16 * t + dc;
          const bool ok = row < j0 && col < k;
          bv[q][t] = U[ok ? static_cast<int64_t>(row) * k + col : 0];
          bv[q][t] = ok ? bv[q][t] : 0.0;
        }
    };
    auto trip = [&](int s0, const double (&bv)[4][4]) {
      double av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) av[q] = -xs[ar * ld + s0 + 4 * q + ak];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[q], bv[q][t], acc[t], 0, 0, 0);
    };
    // two register sets in turn (j0 is a multiple of 64: trips come in fours)
    double b1[4][4];
    load_u(0, bn);
    for (int s0 = 0; s0 < j0; s0 += 32) {
      load_u(s0 + 16, b1);
      trip(s0, bn);
      load_u(s0 + 32, bn);
      trip(s0 + 16, b1);
    }
    // A into LDS (the block's columns of X), then X[:, blk] = A Dinv (upper
    // triangular: tile t takes k < 16 (t + 1))
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) xs[(dr + 4 * v) * ld + j0 + 16 * t + dc] = acc[t][v];
    gq_f64x4 x[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) x[t][v] = 0.0;
    const double* D = Dv + static_cast<int64_t>(jb) * kSolveBlk * kSolveBlk;
#pragma unroll
    for (int s0 = 0; s0 < kSolveBlk; s0 += 16) {
      double av[4], bv[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = xs[ar * ld + j0 + s0 + 4 * q + ak];
#pragma unroll
        for (int t = 0; t < 4; ++t) bv[q][t] = D[(s0 + 4 * q + dr) * kSolveBlk + 16 * t + dc];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (s0 < 16 * (t + 1)) x[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[q], bv[q][t], x[t], 0, 0, 0);
    }
    // X into LDS (over A: this wave's reads of A above come first) and out
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + dr + 4 * v, col = j0 + 16 * t + dc;
        xs[(dr + 4 * v) * ld + j0 + 16 * t + dc] = x[t][v];
        if (row < a.m && col < k) Po[static_cast<int64_t>(row) * k + col] = static_cast<float>(x[t][v]);
      }
  }
}

// ---------------------------------------------------------------------------
// Stage 3 for 224 < k <= kRegRankK (256) (smaller k take the paired version
// below), every value in fp64, one block of 512 threads per matrix, with the
// k x k matrix in registers: thread (tr,
// tc) = (t / 32, t % 32) holds the entries (tr + 16 i, tc + 32 j), i < 16,
// j < 8, of the upper triangle (the slots with j >= i / 2; the rest would lie
// below the diagonal).  A step publishes one row through LDS (two buffers,
// so one barrier per step) and updates whole row blocks without branches:
// rows that must not change get a zero multiplier, and slots outside the
// matrix or below its diagonal take values that nothing reads.  Global
// memory is touched outside the step loop only, and the loop holds no
// division or square root (a dependent fp64 operation costs tens of cycles,
// and the steps form one chain).
//
// Right-looking Cholesky one column at a time, in the form S = L' diag(d)
// L'^T: step p publishes S[p][.], takes d_p = S[p][p] and 1 / d_p
// (the hardware reciprocal and two Newton steps) and subtracts S[p][r]
// S[p][c] / d_p from the entries of the rows r > p.  Row p of the slots
// keeps S[p][.]; at the end U[p][p] = sqrt(d_p) and U[p][c] = S[p][c] /
// sqrt(d_p).  The dead-column rule is the panel kernel's: a dead row p is
// e_p in U and takes nothing from later columns.
// ---------------------------------------------------------------------------
constexpr int kRegT = 512;
constexpr int kRegBR = kRegRankK / 16;  // row blocks of 16
constexpr int kRegBC = kRegRankK / 32;  // column blocks of 32

// 1 / x for a positive normal x: the hardware estimate and two Newton steps.
__device__ __forceinline__ double recip_f64(double x) {
  double y = __builtin_amdgcn_rcp(x);
  double e = fma(-x, y, 1.0);
  y = fma(y, e, y);
  e = fma(-x, y, 1.0);
  return fma(y, e, y);
}

__global__ __launch_bounds__(kRegT) void chol_reg_kernel(CholArgs a) {
  __shared__ double rowbuf[2][kRegRankK];
  __shared__ double diag0[kRegRankK], dval[kRegRankK];
  __shared__ int deads[kRegRankK];
  const int b = blockIdx.x, k = a.k;
  const int tr = threadIdx.x >> 5, tc = threadIdx.x & 31;
  double* U = a.S + static_cast<int64_t>(b) * k * k;
  double s[kRegBR][kRegBC];
#pragma unroll
  for (int i = 0; i < kRegBR; ++i)
#pragma unroll
    for (int j = i >> 1; j < kRegBC; ++j) {
      const int r = tr + 16 * i, c = tc + 32 * j;
      s[i][j] = (r < k && c < k && c >= r) ? U[static_cast<int64_t>(r) * k + c] : 0.0;
    }
  if (threadIdx.x < kRegRankK) {
    const int c = threadIdx.x;
    diag0[c] = c < k ? U[static_cast<int64_t>(c) * k + c] : 0.0;
    rowbuf[0][c] = 0.0;
    rowbuf[1][c] = 0.0;
  }
  __syncthreads();
  for (int p = 0; p < k; ++p) {
    const int pi = p >> 4;
    const int pr = p & 15;
    double* rb = rowbuf[p & 1];
    if (tr == pr) {
      // entries left of p are published as zero, so every slot stays finite
#pragma unroll
      for (int i = 0; i < kRegBR; ++i)
        if (i == pi) {
#pragma unroll
          for (int j = i >> 1; j < kRegBC; ++j) rb[tc + 32 * j] = tc + 32 * j >= p ? s[i][j] : 0.0;
        }
    }
    __syncthreads();
    double uc[kRegBC], ur[kRegBR];
#pragma unroll
    for (int j = 0; j < kRegBC; ++j) uc[j] = rb[tc + 32 * j];
#pragma unroll
    for (int i = 0; i < kRegBR; ++i) ur[i] = rb[tr + 16 * i];
    const double d = rb[p], d0 = diag0[p];
    const bool is_dead = !(d0 > 0.0) || !(d > 1e-12 * d0);
    if (threadIdx.x == 0) {
      dval[p] = d;
      deads[p] = is_dead ? 1 : 0;
    }
    if (!is_dead) {
      const double rd = recip_f64(d);
#pragma unroll
      for (int i = 0; i < kRegBR; ++i) {
        if (i >= pi) {
          // rows up to p keep S[r][.] for the end: a zero multiplier
          const double x = (i > pi || tr > pr) ? ur[i] * rd : 0.0;
#pragma unroll
          for (int j = i >> 1; j < kRegBC; ++j) s[i][j] = fma(-x, uc[j], s[i][j]);
        }
      }
    }
  }
  __syncthreads();
  // U's rows: sqrt(d_r) on the diagonal, S[r][.] / sqrt(d_r) right of it (zero for a dead row)
#pragma unroll
  for (int i = 0; i < kRegBR; ++i) {
    const int r = tr + 16 * i;
    if (r < k) {
      const bool dr = deads[r] != 0;
      const double pv = dr ? 1.0 : sqrt(dval[r]);
      const double iv = 1.0 / pv;
#pragma unroll
      for (int j = i >> 1; j < kRegBC; ++j) {
        const int c = tc + 32 * j;
        if (c >= r && c < k) U[static_cast<int64_t>(r) * k + c] = c == r ? pv : (dr ? 0.0 : s[i][j] * iv);
      }
    }
  }
  if (threadIdx.x < k) a.dead[static_cast<int64_t>(b) * k + threadIdx.x] = deads[threadIdx.x];
}

// k <= 224: the same in pairs of columns, one barrier per pair.  Rows p and
// q = p + 1 are published together; each thread applies row p's update to
// its copies of row q's values (t = S[q][.] - S[p][q] / d_p S[p][.], d_q =
// t[q]) and then both rank-one updates to its slots, so rows below q take
// both terms, row q takes row p's, and rows up to p none.  The slot layout
// is the one above restricted to 14 row blocks and 7 column blocks, which
// leaves registers for both rows' values.
constexpr int kPairK = 224;
constexpr int kPairBR = kPairK / 16, kPairBC = kPairK / 32;

__global__ __launch_bounds__(kRegT) void chol_pair_kernel(CholArgs a) {
  __shared__ double rowbuf[2][2][kPairK];
  __shared__ double diag0[kPairK], dval[kPairK];
  __shared__ int deads[kPairK];
  const int b = blockIdx.x, k = a.k;
  const int tr = threadIdx.x >> 5, tc = threadIdx.x & 31;
  double* U = a.S + static_cast<int64_t>(b) * k * k;
  double s[kPairBR][kPairBC];
#pragma unroll
  for (int i = 0; i < kPairBR; ++i)
#pragma unroll
    for (int j = i >> 1; j < kPairBC; ++j) {
      const int r = tr + 16 * i, c = tc + 32 * j;
      s[i][j] = (r < k && c < k && c >= r) ? U[static_cast<int64_t>(r) * k + c] : 0.0;
    }
  if (threadIdx.x < kPairK) {
    const int c = threadIdx.x;
    diag0[c] = c < k ? U[static_cast<int64_t>(c) * k + c] : 0.0;
#pragma unroll
    for (int x = 0; x < 2; ++x) rowbuf[x][0][c] = rowbuf[x][1][c] = 0.0;
  }
  __syncthreads();
  for (int p = 0; p < k; p += 2) {
    const int q = p + 1;
    const bool two = q < k;
    const int pi = p >> 4, qi = q >> 4;
    double* rb0 = rowbuf[(p >> 1) & 1][0];
    double* rb1 = rowbuf[(p >> 1) & 1][1];
    // entries left of a row's diagonal are published as zero, so every slot stays finite
    if (tr == (p & 15)) {
#pragma unroll
      for (int i = 0; i < kPairBR; ++i)
        if (i == pi) {
#pragma unroll
          for (int j = i >> 1; j < kPairBC; ++j) rb0[tc + 32 * j] = tc + 32 * j >= p ? s[i][j] : 0.0;
        }
    }
    if (two && tr == (q & 15)) {
#pragma unroll
      for (int i = 0; i < kPairBR; ++i)
        if (i == qi) {
#pragma unroll
          for (int j = i >> 1; j < kPairBC; ++j) rb1[tc + 32 * j] = tc + 32 * j >= q ? s[i][j] : 0.0;
        }
    }
    __syncthreads();
    // Only row blocks i >= pi are updated, and their slots use column blocks
    // j >= pi / 2: the published values outside those are not read (the LDS
    // reads, not the FMAs, dominate a step at these sizes).  pi is uniform, so
    // the guards are scalar branches.
    const int pc = pi >> 1;
    double u0c[kPairBC], u1c[kPairBC];
#pragma unroll
    for (int j = 0; j < kPairBC; ++j) {
      u0c[j] = 0.0;
      u1c[j] = 0.0;
      if (j >= pc) {
        u0c[j] = rb0[tc + 32 * j];
        u1c[j] = rb1[tc + 32 * j];
      }
    }
    const double d0 = rb0[p], e0 = diag0[p];
    const bool dead0 = !(e0 > 0.0) || !(d0 > 1e-12 * e0);
    const double r0 = recip_f64(d0);
    const double rd0 = dead0 ? 0.0 : r0;
    double rd1 = 0.0, d1 = 0.0;
    bool dead1 = true;
    if (two) {
      const double f = rb0[q] * rd0;  // S[p][q] / d_p (zero for a dead row p)
      d1 = fma(-f, rb0[q], rb1[q]);
      const double e1 = diag0[q];
      dead1 = !(e1 > 0.0) || !(d1 > 1e-12 * e1);
      const double r1 = recip_f64(d1);
      rd1 = dead1 ? 0.0 : r1;
#pragma unroll
      for (int j = 0; j < kPairBC; ++j) u1c[j] = fma(-f, u0c[j], u1c[j]);
    }
    const double fq = two ? rb0[q] * rd0 : 0.0;  // the same f, for the row values read below
    if (threadIdx.x == 0) {
      dval[p] = d0;
      deads[p] = dead0 ? 1 : 0;
      if (two) {
        dval[q] = d1;
        deads[q] = dead1 ? 1 : 0;
      }
    }
#pragma unroll
    for (int i = 0; i < kPairBR; ++i) {
      if (i >= pi) {
        const int r = tr + 16 * i;
        const double u0r = rb0[r], u1r = fma(-fq, u0r, rb1[r]);
        const double x0 = r > p ? u0r * rd0 : 0.0;
        const double x1 = r > q ? u1r * rd1 : 0.0;
#pragma unroll
        for (int j = i >> 1; j < kPairBC; ++j) s[i][j] = fma(-x1, u1c[j], fma(-x0, u0c[j], s[i][j]));
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPairBR; ++i) {
    const int r = tr + 16 * i;
    if (r < k) {
      const bool dr = deads[r] != 0;
      const double pv = dr ? 1.0 : sqrt(dval[r]);
      const double iv = 1.0 / pv;
#pragma unroll
      for (int j = i >> 1; j < kPairBC; ++j) {
        const int c = tc + 32 * j;
        if (c >= r && c < k) U[static_cast<int64_t>(r) * k + c] = c == r ? pv : (dr ? 0.0 : s[i][j] * iv);
      }
    }
  }
  if (threadIdx.x < k) a.dead[static_cast<int64_t>(b) * k + threadIdx.x] = deads[threadIdx.x];
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

hipError_t launch_col_norms(const UnitArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(colsq_kernel, dim3(a.nchunk, batch), dim3(kGT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colinv_kernel, dim3(batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_codes_t(const void* const* codes, int n, int k, uint16_t* ct, int64_t s_ct, int batch,
                          hipStream_t s) {
  const dim3 g((k + 63) / 64, (n + 63) / 64, batch);
  hipLaunchKernelGGL(codes_t_kernel, g, dim3(kGT), 0, s, codes, n, k, ct, s_ct);
  return hipGetLastError();
}

hipError_t launch_mq(const MQArgs& a, int batch, hipStream_t s) {
  const dim3 g((a.N + kTT - 1) / kTT, (a.M + kTT - 1) / kTT, batch * a.pieces);
  hipLaunchKernelGGL(mq_kernel, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tall(const TallArgs& a, int batch, hipStream_t s) {
  if (a.Bh == nullptr || a.Bl == nullptr) return hipErrorInvalidValue;  // B comes pre-split
  const dim3 g((a.N + kTT - 1) / kTT, (a.M + kTT - 1) / kTT, batch * a.pieces);
  hipLaunchKernelGGL(tall_gemm_kernel, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_t(const float* X, int64_t sX, int rows, int k, uint16_t* hi, uint16_t* lo, int64_t sT,
                          int batch, hipStream_t s) {
  const dim3 g((k + 63) / 64, (rows + 63) / 64, batch);
  hipLaunchKernelGGL(split_t_kernel, g, dim3(kGT), 0, s, X, sX, rows, k, hi, lo, sT);
  return hipGetLastError();
}

hipError_t launch_split(const float* X, int64_t sX, int64_t count, uint16_t* hi, uint16_t* lo, int64_t sT, int batch,
                        hipStream_t s) {
  int64_t blocks = (count + kGT - 1) / kGT;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(split_kernel, dim3(static_cast<unsigned>(blocks), batch), dim3(kGT), 0, s, X, sX, count, hi, lo,
                     sT);
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
  if (a.g_dtype == 0) hipLaunchKernelGGL(recon_kernel<0>, g, dim3(kGT), 0, s, a);
  else if (a.g_dtype == 1) hipLaunchKernelGGL(recon_kernel<1>, g, dim3(kGT), 0, s, a);
  else hipLaunchKernelGGL(recon_kernel<2>, g, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_residual(const ResidualArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(residual_kernel, grid_blocks(a.rows, a.cols, batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gram(const CholArgs& a, int batch, hipStream_t s) {
  if (a.k <= kRegRankK) {
    const int nbk = (a.k + 15) / 16, npairs = nbk * (nbk + 1) / 2;
    const dim3 grid(a.nchunk, (npairs + kGramPairsPerPass - 1) / kGramPairsPerPass, batch);
    hipLaunchKernelGGL(gram_mfma_kernel, grid, dim3(kGT), 0, s, a);
  } else {
    hipLaunchKernelGGL(gram64_kernel, dim3(a.nchunk, batch), dim3(kGT),
                       static_cast<size_t>(kGramRows) * a.k * sizeof(double), s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = (static_cast<int64_t>(a.k) * a.k + kGT - 1) / kGT;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gram_sum_kernel, dim3(static_cast<unsigned>(blocks), batch), dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chol(const CholArgs& a, int batch, hipStream_t s) {
  if (a.k <= kPairK) {
    hipLaunchKernelGGL(chol_pair_kernel, dim3(batch), dim3(kRegT), 0, s, a);
    return hipGetLastError();
  }
  if (a.k <= kRegRankK) {
    hipLaunchKernelGGL(chol_reg_kernel, dim3(batch), dim3(kRegT), 0, s, a);
    return hipGetLastError();
  }
  CholArgs c = a;
  c.panel = 32;
  while (c.panel > 1 && c.panel * a.k > kPanelElems) c.panel >>= 1;
  hipLaunchKernelGGL(chol_panel_kernel, dim3(batch), dim3(kGT), static_cast<size_t>(c.panel) * a.k * sizeof(double), s,
                     c);
  return hipGetLastError();
}

hipError_t launch_row_solve(const CholArgs& a, int batch, hipStream_t s) {
  const int nbk = (a.k + kSolveBlk - 1) / kSolveBlk;
  hipLaunchKernelGGL(diag_inv_kernel, dim3(nbk, batch), dim3(kSolveBlk), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = static_cast<size_t>(16) * (kSolveBlk * nbk + 1) * sizeof(double);  // <= 131 KB (k <= 1024)
  hipLaunchKernelGGL(row_solve_mfma_kernel, dim3((a.m + 15) / 16, batch), dim3(64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_ptr_table(float* base, int64_t stride, int batch, float** out, hipStream_t s) {
  hipLaunchKernelGGL(ptr_table_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, base, stride, batch, out);
  return hipGetLastError();
}

}  // namespace muon
