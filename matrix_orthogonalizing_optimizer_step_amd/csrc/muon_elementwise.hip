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
constexpr int kNormThreads = 256;  // momentum/norm kernel (1024 measured 1 % faster, within noise)

// Eight consecutive elements of dtype D as fp64 (16- or 32-byte loads).
template <int D>
__device__ __forceinline__ void load8(const void* p, int64_t i, double (&v)[8]) {
  if constexpr (D == kF32) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 x = q[0], y = q[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = static_cast<uint16_t>(w[k] & 0xffffu), hi = static_cast<uint16_t>(w[k] >> 16);
      v[2 * k] = D == kBF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
      v[2 * k + 1] = D == kBF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
  }
}

// Eight consecutive elements of dtype D as loaded (no conversion), so a
// chunk can be in flight while the previous one is converted and stored.
template <int D>
struct Raw8 {
  uint4 v[D == kF32 ? 2 : 1];
};
template <int D>
__device__ __forceinline__ Raw8<D> load_raw8(const void* p, int64_t i) {
  Raw8<D> r;
  const uint4* q = reinterpret_cast<const uint4*>(static_cast<const char*>(p) + i * (D == kF32 ? 4 : 2));
#pragma unroll
  for (int k = 0; k < (D == kF32 ? 2 : 1); ++k) r.v[k] = q[k];
  return r;
}
template <int D>
__device__ __forceinline__ void raw8_to_f64(const Raw8<D>& r, double (&v)[8]) {
  if constexpr (D == kF32) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      v[4 * k] = __uint_as_float(r.v[k].x);
      v[4 * k + 1] = __uint_as_float(r.v[k].y);
      v[4 * k + 2] = __uint_as_float(r.v[k].z);
      v[4 * k + 3] = __uint_as_float(r.v[k].w);
    }
  } else {
    const uint32_t w[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = static_cast<uint16_t>(w[k] & 0xffffu), hi = static_cast<uint16_t>(w[k] >> 16);
      v[2 * k] = D == kBF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
      v[2 * k + 1] = D == kBF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
  }
}

// Round eight fp64 values once into the state dtype D (f32 or bf16), store
// them with 16-byte stores and add the squares of the stored values to ss.
template <int D>
__device__ __forceinline__ void round_store8(void* p, int64_t i, const double (&x)[8], double& ss) {
  if constexpr (D == kF32) {
    float f[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      f[k] = static_cast<float>(x[k]);
      ss = fma(static_cast<double>(f[k]), static_cast<double>(f[k]), ss);
    }
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + i);
    q[0] = make_float4(f[0], f[1], f[2], f[3]);
    q[1] = make_float4(f[4], f[5], f[6], f[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = f64_to_bf16(x[2 * k]), hi = f64_to_bf16(x[2 * k + 1]);
      const double a = bf16_to_f32(lo), b = bf16_to_f32(hi);
      ss = fma(a, a, ss);
      ss = fma(b, b, ss);
      w[k] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ double load1(const void* p, int64_t i, int d) {
  return static_cast<double>(load_as_f32(p, i, d));
}

// Round an fp64 value into dtype d (f32 or bf16); returns the stored value.
__device__ __forceinline__ double store1(void* p, int64_t i, int d, double x) {
  if (d == kF32) {
    const float f = static_cast<float>(x);
    static_cast<float*>(p)[i] = f;
    return f;
  }
  const uint16_t h = f64_to_bf16(x);
  static_cast<uint16_t*>(p)[i] = h;
  return bf16_to_f32(h);
}

template <int NT = kThreads>
__device__ __forceinline__ double block_sum(double x, double* red) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

// One fp64 partial sum of squares per block over a fixed chunk of the matrix;
// in momentum mode (G given) the chunk is first updated and written back.
template <int D>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(NormArgs a) {
  __shared__ double red[kNormThreads / 64];
  const int b = blockIdx.y;
  if (blockIdx.x == 0 && b == 0)
    for (int i = threadIdx.x; i < a.nzero; i += kNormThreads) a.zero[i] = 0;
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
    const int64_t i0 = start + 8 * static_cast<int64_t>(threadIdx.x), step = 8 * kNormThreads;
    if (Gp != nullptr) {
      if constexpr (D != kF16) {  // state dtypes are f32 or bf16
        // The next chunk's loads go out before this chunk's stores: M is
        // updated in place, and a store issued ahead of a load would hold the
        // wait for that load's data behind the store's completion.
        Raw8<D> rm, rg;
        if (i0 < vec_end) {
          rm = load_raw8<D>(Mp, i0);
          rg = load_raw8<D>(Gp, i0);
        }
        for (int64_t i = i0; i < vec_end; i += step) {
          const Raw8<D> cm = rm, cg = rg;
          if (i + step < vec_end) {
            rm = load_raw8<D>(Mp, i + step);
            rg = load_raw8<D>(Gp, i + step);
          }
          double m[8], g[8], x[8];
          raw8_to_f64<D>(cm, m);
          raw8_to_f64<D>(cg, g);
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = fma(a.mu, m[k], g[k]);
          round_store8<D>(Wp, i, x, ss);
        }
      }
    } else {
      for (int64_t i = i0; i < vec_end; i += step) {
        double m[8];
        load8<D>(Mp, i, m);
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fma(m[k], m[k], ss);
      }
    }
  }
  for (int64_t i = vec_end + threadIdx.x; i < end; i += kNormThreads) {
    double m = load1(Mp, i, D);
    if (Gp != nullptr) m = store1(Wp, i, D, fma(a.mu, m, load1(Gp, i, D)));
    ss = fma(m, m, ss);
  }
  ss = block_sum<kNormThreads>(ss, red);
  if (threadIdx.x == 0) a.partials[static_cast<int64_t>(b) * kNormBlocks + blockIdx.x] = ss;
}

// The scale 1 / (||M||_F + eps) of matrix b from its kNormBlocks partials,
// summed in a fixed order.  All threads of the block must call this.
__device__ __forceinline__ float block_scale(const PrepArgs& a, int b, double* red) {
  double ss = 0.0;
  for (int p = threadIdx.x; p < kNormBlocks; p += kThreads) ss += a.partials[static_cast<int64_t>(b) * kNormBlocks + p];
  ss = block_sum(ss, red);
  return static_cast<float>(1.0 / (sqrt(ss) + a.eps));
}

// 16-bit operands: X0 = M / (||M||_F + eps) for one 64 x 64 tile of X (rows
// i0.., columns j0..), with X = M or M^T.  The tile is read from M with
// 16-byte loads where the rows allow it, rounded, and kept in LDS as X and
// X^T (16-bit, rows padded to 72 elements); then each of X and X^T is written
// as 8 whole 1 KB fragments of the packed operand layout (two 32-row blocks
// x four 16-column k-steps), one 16-byte store per lane.
constexpr int kPT = 64;        // tile edge
constexpr int kPL = kPT + 8;   // LDS row length (elements)

template <int D, int OP>
__global__ __launch_bounds__(kThreads) void prep_packed_kernel(PrepArgs a) {
  using O = OpT<OP>;
  __shared__ __align__(16) uint16_t xn[kPT * kPL];  // X tile, row-major
  __shared__ __align__(16) uint16_t xt[kPT * kPL];  // X^T tile, row-major
  __shared__ double red[kThreads / 64];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * kPT, j0 = blockIdx.x * kPT;
  const float s = block_scale(a, b, red);
  const void* Mp = a.M[b];
  // The tile covers M rows u0.., columns v0.. (u = i, v = j, or swapped).
  const int u0 = a.transposed ? j0 : i0, v0 = a.transposed ? i0 : j0;
  const bool vec = (reinterpret_cast<uintptr_t>(Mp) & 15u) == 0 && (a.cols & 7) == 0;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = threadIdx.x + pass * kThreads;  // chunk of 8 elements: M row u0 + c / 8, columns 8 (c % 8)..
    const int ur = c >> 3, vc = (c & 7) * 8;
    const int u = u0 + ur, v = v0 + vc;
    float x[8];
    if (vec && u < a.rows && v + 8 <= a.cols) {
      double d[8];
      load8<D>(Mp, static_cast<int64_t>(u) * a.cols + v, d);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = static_cast<float>(d[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        x[k] = (u < a.rows && v + k < a.cols) ? load_as_f32(Mp, static_cast<int64_t>(u) * a.cols + v + k, D) : 0.0f;
    }
    uint16_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = O::from_f(x[k] * s);
    // M[u][v + k] is X[u][v + k] (not transposed) or X[v + k][u]
    uint16_t* row = a.transposed ? xt : xn;  // the tile whose rows run along M's rows
    uint16_t* col = a.transposed ? xn : xt;
    *reinterpret_cast<uint4*>(row + ur * kPL + vc) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
#pragma unroll
    for (int k = 0; k < 8; ++k) col[(vc + k) * kPL + ur] = h[k];
  }
  __syncthreads();
  // fragment f = 4 * (row block) + (k-step); lane L holds row 32 rb + L % 32,
  // columns 16 ks + 8 (L / 32) .. + 7
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int f = (threadIdx.x >> 6) + 4 * pass;
    const int rb = f >> 2, ks = f & 3;
    const int r = 32 * rb + (lane & 31), k = 16 * ks + 8 * (lane >> 5);
    const uint4 vn = *reinterpret_cast<const uint4*>(xn + r * kPL + k);
    const uint4 vt = *reinterpret_cast<const uint4*>(xt + r * kPL + k);
    uint16_t* XN = static_cast<uint16_t*>(a.XN) + static_cast<int64_t>(b) * a.sXN;
    uint16_t* XT = static_cast<uint16_t*>(a.XT) + static_cast<int64_t>(b) * a.sXT;
    *reinterpret_cast<uint4*>(XN + op_index<OP>(i0 + 32 * rb, j0 + 16 * ks, a.m_pad) + 8 * lane) = vn;
    *reinterpret_cast<uint4*>(XT + op_index<OP>(j0 + 32 * rb, i0 + 16 * ks, a.n_pad) + 8 * lane) = vt;
  }
}

// fp32 check path: X0 in fp32, row-major, X (n_pad x m_pad) and X^T
// (m_pad x n_pad) with zero padding; one 64 x 64 tile per block, staged
// through LDS so both layouts are written with coalesced stores.
template <int D>
__global__ __launch_bounds__(kThreads) void prep_f32_kernel(PrepArgs a) {
  __shared__ float tile[64][65];
  __shared__ double red[kThreads / 64];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const float s = block_scale(a, b, red);
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
  float* XN = static_cast<float*>(a.XN) + static_cast<int64_t>(b) * a.sXN;
  float* XT = static_cast<float*>(a.XT) + static_cast<int64_t>(b) * a.sXT;
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int r = e >> 6, c = e & 63;
    XN[static_cast<int64_t>(i0 + r) * a.m_pad + j0 + c] = a.transposed ? tile[c][r] : tile[r][c];
    XT[static_cast<int64_t>(j0 + r) * a.n_pad + i0 + c] = a.transposed ? tile[r][c] : tile[c][r];
  }
}

}  // namespace

hipError_t launch_norm(const NormArgs& a, int batch, hipStream_t s) {
  dim3 grid(kNormBlocks, batch), block(kNormThreads);
  switch (a.m_dtype) {
    case kF32: hipLaunchKernelGGL(norm_kernel<kF32>, grid, block, 0, s, a); break;
    case kBF16: hipLaunchKernelGGL(norm_kernel<kBF16>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(norm_kernel<kF16>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int OP>
static void launch_prep_packed(const PrepArgs& a, int batch, hipStream_t s) {
  const dim3 grid(a.m_pad / kPT, a.n_pad / kPT, batch), block(kThreads);
  switch (a.m_dtype) {
    case kF32: hipLaunchKernelGGL((prep_packed_kernel<kF32, OP>), grid, block, 0, s, a); break;
    case kBF16: hipLaunchKernelGGL((prep_packed_kernel<kBF16, OP>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((prep_packed_kernel<kF16, OP>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_prep(const PrepArgs& a, int batch, int op, hipStream_t s) {
  if (op == kOpBF16) {
    launch_prep_packed<kOpBF16>(a, batch, s);
  } else if (op == kOpF16) {
    launch_prep_packed<kOpF16>(a, batch, s);
  } else {
    const dim3 grid(a.m_pad / 64, a.n_pad / 64, batch), block(kThreads);
    switch (a.m_dtype) {
      case kF32: hipLaunchKernelGGL(prep_f32_kernel<kF32>, grid, block, 0, s, a); break;
      case kBF16: hipLaunchKernelGGL(prep_f32_kernel<kBF16>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(prep_f32_kernel<kF16>, grid, block, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace muon
