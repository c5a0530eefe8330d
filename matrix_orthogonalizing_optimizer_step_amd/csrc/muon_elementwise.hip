// Bandwidth-bound kernels of the Muon step: the momentum update with the
// Frobenius-norm reduction, and the preparation of the normalised 16-bit
// iterate X0 in both layouts.
//
// Momentum ([GRASP framework], [GNS §1.1 eq.(1)]): M <- mu M + G, computed
// as one fp64 fused multiply-add on the exact stored values and rounded once
// (to nearest even) into the state dtype.  The same pass accumulates the sum
// of squares of the stored values for X0 = M / (||M||_F + eps) ([GNS §2.3
// Alg.1]); every block writes one fp64 partial, and the consumer sums a fixed
// list of partials, so the result is bitwise reproducible.
#include "muon_convert.h"
#include "muon_internal.h"

namespace muon {

namespace {

constexpr int kThreads = 256;

template <int D> struct Vec8;
template <> struct Vec8<kF32> {
  static __device__ __forceinline__ void load(const void* p, int64_t i, double* v) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 x = q[0], y = q[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  }
};
template <int D> struct Vec8Half {
  static __device__ __forceinline__ void load(const void* p, int64_t i, double* v) {
    const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = static_cast<uint16_t>(w[k] & 0xffffu), hi = static_cast<uint16_t>(w[k] >> 16);
      v[2 * k] = D == kBF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
      v[2 * k + 1] = D == kBF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
  }
};
template <> struct Vec8<kBF16> : Vec8Half<kBF16> {};
template <> struct Vec8<kF16> : Vec8Half<kF16> {};

__device__ __forceinline__ double load1(const void* p, int64_t i, int d) {
  return static_cast<double>(load_as_f32(p, i, d));
}

// Round an fp64 value into dtype d; returns the stored value as fp64.
__device__ __forceinline__ double store1(void* p, int64_t i, int d, double x) {
  if (d == kF32) {
    const float f = static_cast<float>(x);
    static_cast<float*>(p)[i] = f;
    return f;
  }
  const uint16_t h = f64_to_bf16(x);  // state dtypes are f32 or bf16
  static_cast<uint16_t*>(p)[i] = h;
  return bf16_to_f32(h);
}

__device__ __forceinline__ double block_sum(double x, double* red) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < kThreads / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

template <int D>
__global__ __launch_bounds__(kThreads) void norm_kernel(NormArgs a) {
  __shared__ double red[kThreads / 64];
  const int b = blockIdx.y;
  const void* Mp = a.M[b];
  const void* Gp = a.G != nullptr ? a.G[b] : nullptr;
  void* Wp = a.Mw != nullptr ? a.Mw[b] : nullptr;
  int64_t per = (a.count + kNormBlocks - 1) / kNormBlocks;
  per = (per + 7) & ~static_cast<int64_t>(7);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t end = start + per < a.count ? start + per : a.count;
  double ss = 0.0;
  const bool aligned = ((reinterpret_cast<uintptr_t>(Mp) | reinterpret_cast<uintptr_t>(Gp) |
                         reinterpret_cast<uintptr_t>(Wp)) & 15u) == 0;
  int64_t vec_end = start;
  if (aligned && end > start) {
    vec_end = start + ((end - start) & ~static_cast<int64_t>(7));
    for (int64_t i = start + 8 * static_cast<int64_t>(threadIdx.x); i < vec_end; i += 8 * kThreads) {
      double m[8];
      Vec8<D>::load(Mp, i, m);
      if (Gp != nullptr) {
        double g[8];
        Vec8<D>::load(Gp, i, g);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const double s = store1(Wp, i + k, D, fma(a.mu, m[k], g[k]));
          ss = fma(s, s, ss);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fma(m[k], m[k], ss);
      }
    }
  }
  for (int64_t i = vec_end + threadIdx.x; i < end; i += kThreads) {
    double m = load1(Mp, i, D);
    if (Gp != nullptr) m = store1(Wp, i, D, fma(a.mu, m, load1(Gp, i, D)));
    ss = fma(m, m, ss);
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) a.partials[static_cast<int64_t>(b) * kNormBlocks + blockIdx.x] = ss;
}

// X0 = M / (||M||_F + eps) rounded to the operand type, written as X (n_pad x
// m_pad) and X^T (m_pad x n_pad) in the operand layout (op_index) with zero
// padding.  X = M, or M^T when the
// user matrix has more rows than columns.  One 64 x 64 tile per block, staged
// through LDS so both layouts are written with coalesced stores.
template <int D, int OP>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
  using O = OpT<OP>;
  using T = typename O::T;
  __shared__ float tile[64][65];
  __shared__ double red[kThreads / 64];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  double ss = 0.0;
  for (int p = threadIdx.x; p < kNormBlocks; p += kThreads) ss += a.partials[static_cast<int64_t>(b) * kNormBlocks + p];
  ss = block_sum(ss, red);
  const float s = static_cast<float>(1.0 / (sqrt(ss) + a.eps));
  const void* Mp = a.M[b];
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int r = e >> 6, c = e & 63;
    float x = 0.0f;
    if (!a.transposed) {  // tile[r][c] = X[i0 + r][j0 + c] = M[i][j]
      const int i = i0 + r, j = j0 + c;
      if (i < a.n && j < a.m) x = load_as_f32(Mp, static_cast<int64_t>(i) * a.cols + j, D);
    } else {              // tile[r][c] = X[i0 + c][j0 + r] = M[j0 + r][i0 + c]
      const int j = j0 + r, i = i0 + c;
      if (i < a.n && j < a.m) x = load_as_f32(Mp, static_cast<int64_t>(j) * a.cols + i, D);
    }
    tile[r][c] = x * s;
  }
  __syncthreads();
  T* XN = static_cast<T*>(a.XN) + static_cast<int64_t>(b) * a.sXN;
  T* XT = static_cast<T*>(a.XT) + static_cast<int64_t>(b) * a.sXT;
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int r = e >> 6, c = e & 63;
    // X[i0 + r][j0 + c]
    const float xn = a.transposed ? tile[c][r] : tile[r][c];
    XN[op_index<OP>(i0 + r, j0 + c, a.m_pad)] = O::from_f(xn);
    // X^T[j0 + r][i0 + c] = X[i0 + c][j0 + r]
    const float xt = a.transposed ? tile[r][c] : tile[c][r];
    XT[op_index<OP>(j0 + r, i0 + c, a.n_pad)] = O::from_f(xt);
  }
}

}  // namespace

hipError_t launch_norm(const NormArgs& a, int batch, hipStream_t s) {
  dim3 grid(kNormBlocks, batch), block(kThreads);
  switch (a.m_dtype) {
    case kF32: hipLaunchKernelGGL(norm_kernel<kF32>, grid, block, 0, s, a); break;
    case kBF16: hipLaunchKernelGGL(norm_kernel<kBF16>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(norm_kernel<kF16>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int OP>
static void launch_prep_op(const PrepArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.m_pad / 64, a.n_pad / 64, batch), block(kThreads);
  switch (a.m_dtype) {
    case kF32: hipLaunchKernelGGL((prep_kernel<kF32, OP>), grid, block, 0, s, a); break;
    case kBF16: hipLaunchKernelGGL((prep_kernel<kBF16, OP>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((prep_kernel<kF16, OP>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_prep(const PrepArgs& a, int batch, int op, hipStream_t s) {
  if (op == kOpBF16) launch_prep_op<kOpBF16>(a, batch, s);
  else if (op == kOpF16) launch_prep_op<kOpF16>(a, batch, s);
  else launch_prep_op<kOpF32>(a, batch, s);
  return hipGetLastError();
}

}  // namespace muon
