// Batched GEMM kernels for the Newton-Schulz iterations, with fused epilogues.
//
// Every product of the standard and Gram Newton-Schulz iterations ([GNS §1.2]
// and [GNS §2.3-3.4] of the Gram Newton-Schulz notes) is written in the
// "NT" form C[i][j] = sum_k P[i][k] Q[j][k] with both operands contiguous
// along k:
//   X X^T            P = Q = X (n x m)                      symmetric
//   A A, R R, Q Z,   P, Q symmetric n x n (Q^T = Q)         symmetric
//   R Z, Z (RZ)
//   B X, Q X         P = B or Q (n x n), Q = X^T (m x n)    general
// X is kept in both layouts (X and X^T) by the producing epilogue, so one
// tile loop serves every product.  Symmetric products compute only the tiles
// on or below the diagonal and store each value at (i, j) and (j, i), the
// triangle-only scheme the notes describe for their symmetric GEMM [GNS §4].
//
// 16-bit operands run on CDNA4 MFMA (v_mfma_f32_32x32x16_{bf16,f16}) with
// fp32 accumulation; the fp32 check path accumulates fp32 operands in fp64.
#include "muon_convert.h"
#include "muon_internal.h"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Tile t of the lower triangle (row-major over rows I, J <= I).
__device__ __forceinline__ void tri_tile(int t, int& I, int& J) {
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  I = i;
  J = t - i * (i + 1) / 2;
}

struct EpiState {
  float alpha, beta, gamma, ap;
  double tr, ss;
};

// The diagonal shift a' of matrix b: mean of a + b l + c l^2 over the
// eigenvalues l of the Gram matrix, from its trace and Frobenius norm (both
// reduced from per-tile partials in a fixed order, so every block of a
// launch gets the same value).  All threads of the block must call this.
template <int NT>
__device__ float block_shift(const GemmArgs& a, int b, double* red) {
  if (a.part_in != nullptr) {
    double tr = 0.0, ss = 0.0;
    const double* p = a.part_in + static_cast<int64_t>(b) * a.npart_in * 2;
    for (int i = threadIdx.x; i < a.npart_in; i += NT) {
      tr += p[2 * i];
      ss += p[2 * i + 1];
    }
    for (int off = 32; off > 0; off >>= 1) {
      tr += __shfl_xor(tr, off);
      ss += __shfl_xor(ss, off);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      red[2 * w] = tr;
      red[2 * w + 1] = ss;
    }
    __syncthreads();
    double T = 0.0, S = 0.0;
    for (int i = 0; i < NT / 64; ++i) {
      T += red[2 * i];
      S += red[2 * i + 1];
    }
    __syncthreads();
    const double n = static_cast<double>(a.n_real);
    return static_cast<float>(a.coef_a + a.coef_b * (T / n) + a.coef_c * (S / n));
  }
  if (a.shift_in != nullptr) return a.shift_in[b];
  return a.coef_a;
}

template <int NT>
__device__ void block_init(const GemmArgs& a, int b, int tile, double* red, EpiState& st) {
  st.ap = block_shift<NT>(a, b, red);
  if (a.shift_out != nullptr && tile == 0 && threadIdx.x == 0) a.shift_out[b] = st.ap;
  st.alpha = a.alpha_c + a.alpha_a * st.ap;
  st.beta = a.beta_c + a.beta_a * st.ap;
  st.gamma = a.gamma_c + a.gamma_a * st.ap;
  st.tr = 0.0;
  st.ss = 0.0;
}

// Write the (trace, sum of squares) partial of this tile.
template <int NT>
__device__ void block_partials(const GemmArgs& a, int b, int tile, double* red, EpiState& st) {
  if (a.part_out == nullptr) return;
  double tr = st.tr, ss = st.ss;
  for (int off = 32; off > 0; off >>= 1) {
    tr += __shfl_xor(tr, off);
    ss += __shfl_xor(ss, off);
  }
  __syncthreads();
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = tr;
    red[2 * w + 1] = ss;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double T = 0.0, S = 0.0;
    for (int i = 0; i < NT / 64; ++i) {
      T += red[2 * i];
      S += red[2 * i + 1];
    }
    double* o = a.part_out + (static_cast<int64_t>(b) * a.ntiles + tile) * 2;
    o[0] = T;
    o[1] = S;
  }
}

// Epilogue for one element (i, j) of matrix b; for symmetric products the
// caller only passes i >= j and the value is mirrored to (j, i).
template <int OP>
__device__ __forceinline__ void epi_elem(const GemmArgs& a, int b, int i, int j, float acc,
                                         EpiState& st) {
  using O = OpT<OP>;
  using T = typename O::T;
  float e = 0.0f;
  const int64_t ie = static_cast<int64_t>(b) * a.sE + static_cast<int64_t>(i) * a.lde + j;
  if (a.E32 != nullptr) {
    e = a.E32[ie];
  } else if (a.E16 != nullptr) {
    e = O::to_f(static_cast<const T*>(a.E16)[ie]);
  }
  const bool diag = (i == j) && (i < a.n_real);
  float v = st.alpha * acc + st.beta * e;
  if (diag) v += st.gamma;
  if (a.final_mode) {
    if (i < a.n_real && j < a.m_real) {
      const int64_t idx = a.transposed ? static_cast<int64_t>(j) * a.user_ld + i
                                       : static_cast<int64_t>(i) * a.user_ld + j;
      if (a.W != nullptr) {
        void* w = a.W[b];
        const float wv = load_as_f32(w, idx, a.w_dtype);
        store_from_f32(w, idx, a.w_dtype, wv - a.lr * (v + a.wd * wv));
      }
      if (a.Oout != nullptr) store_from_f32(a.Oout[b], idx, a.o_dtype, v);
    }
    return;
  }
  const bool mirror = a.sym && (i != j);
  const int64_t o = static_cast<int64_t>(b) * a.sO + static_cast<int64_t>(i) * a.ldo + j;
  const int64_t oT = static_cast<int64_t>(b) * a.sO + static_cast<int64_t>(j) * a.ldo + i;
  if (a.out32 != nullptr) {
    a.out32[o] = v;
    if (mirror) a.out32[oT] = v;
  }
  if (a.out16 != nullptr) {
    const T h = O::from_f(v);
    static_cast<T*>(a.out16)[o] = h;
    if (mirror) static_cast<T*>(a.out16)[oT] = h;
  }
  if (a.q32 != nullptr || a.q16 != nullptr) {
    const float q = diag ? v + st.ap : v;
    if (a.q32 != nullptr) {
      a.q32[o] = q;
      if (mirror) a.q32[oT] = q;
    }
    if (a.q16 != nullptr) {
      const T h = O::from_f(q);
      static_cast<T*>(a.q16)[o] = h;
      if (mirror) static_cast<T*>(a.q16)[oT] = h;
    }
  }
  if (a.outT16 != nullptr) {
    static_cast<T*>(a.outT16)[static_cast<int64_t>(b) * a.sOT + static_cast<int64_t>(j) * a.ldot + i] =
        O::from_f(v);
  }
  if (a.part_out != nullptr && i < a.n_real && j < a.n_real) {
    if (diag) st.tr += v;
    st.ss += static_cast<double>(v) * v * (mirror ? 2.0 : 1.0);
  }
}

__device__ __forceinline__ void tile_coords(const GemmArgs& a, int BM, int BN, int& I, int& J) {
  if (a.sym) {
    tri_tile(blockIdx.x, I, J);
  } else {
    const int ntn = a.Ndim / BN;
    I = blockIdx.x / ntn;
    J = blockIdx.x % ntn;
  }
}

// ---------------------------------------------------------------------------
// 16-bit MFMA kernel: 128 x 128 block tile, BK = 64, 4 waves of 64 x 64 each
// (2 x 2 MFMA 32x32x16 tiles per wave).  Operand tiles are staged in LDS with
// a register prefetch of the next k-slab and two LDS stages; 16-byte chunks
// are XOR-swizzled across rows so fragment reads do not hit one bank group.
// ---------------------------------------------------------------------------
template <int OP>
__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  if constexpr (OP == kOpBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 64, kCH = kBK / 8;

__device__ __forceinline__ int swz(int r, int c) { return r * kCH + (c ^ (r & 7)); }

template <int OP>
__global__ __launch_bounds__(256) void gemm_nt_mfma(GemmArgs a) {
  using T = uint16_t;
  __shared__ uint4 smem[2][(kBM + kBN) * kCH];
  __shared__ double red[16];
  const int b = blockIdx.y;
  int I, J;
  tile_coords(a, kBM, kBN, I, J);
  EpiState st;
  block_init<256>(a, b, blockIdx.x, red, st);

  const T* Pb = static_cast<const T*>(a.P) + static_cast<int64_t>(b) * a.sP +
                static_cast<int64_t>(I) * kBM * a.ldp;
  const T* Qb = static_cast<const T*>(a.Q) + static_cast<int64_t>(b) * a.sQ +
                static_cast<int64_t>(J) * kBN * a.ldq;
  const int tid = threadIdx.x;
  const int lrow = tid >> 3;  // 0..31
  const int lch = tid & 7;    // 16-byte chunk within the 64-element k-slab
  uint4 rp[kBM / 32], rq[kBN / 32];

  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < kBM / 32; ++r)
      rp[r] = *reinterpret_cast<const uint4*>(Pb + static_cast<int64_t>(lrow + 32 * r) * a.ldp + k0 + lch * 8);
#pragma unroll
    for (int r = 0; r < kBN / 32; ++r)
      rq[r] = *reinterpret_cast<const uint4*>(Qb + static_cast<int64_t>(lrow + 32 * r) * a.ldq + k0 + lch * 8);
  };
  auto sstore = [&](int stage) {
    uint4* sP = smem[stage];
    uint4* sQ = smem[stage] + kBM * kCH;
#pragma unroll
    for (int r = 0; r < kBM / 32; ++r) sP[swz(lrow + 32 * r, lch)] = rp[r];
#pragma unroll
    for (int r = 0; r < kBN / 32; ++r) sQ[swz(lrow + 32 * r, lch)] = rq[r];
  };

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;

  const int nk = a.K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const uint4* sP = smem[cur];
    const uint4* sQ = smem[cur] + kBM * kCH;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      uint4 af[2], bf[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[mi] = sP[swz(wm * 64 + mi * 32 + (lane & 31), c)];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bf[ni] = sQ[swz(wn * 64 + ni * 32 + (lane & 31), c)];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32<OP>(af[mi], bf[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // MFMA 32x32 result layout: lane l, register v hold row 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = I * kBM + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int j = J * kBN + wn * 64 + ni * 32 + (lane & 31);
        if (a.sym && i < j) continue;
        epi_elem<OP>(a, b, i, j, acc[mi][ni][v], st);
      }
  block_partials<256>(a, b, blockIdx.x, red, st);
}

// ---------------------------------------------------------------------------
// fp32 check path: fp32 operands, exact products and fp64 accumulation.
// 64 x 64 block tile, 16 x 16 threads with 4 x 4 outputs each.  Slow.
// ---------------------------------------------------------------------------
constexpr int kCB = 64;

__global__ __launch_bounds__(256) void gemm_nt_f64acc(GemmArgs a) {
  __shared__ float sP[16][kCB + 1];
  __shared__ float sQ[16][kCB + 1];
  __shared__ double red[16];
  const int b = blockIdx.y;
  int I, J;
  tile_coords(a, kCB, kCB, I, J);
  EpiState st;
  block_init<256>(a, b, blockIdx.x, red, st);
  const float* Pb = static_cast<const float*>(a.P) + static_cast<int64_t>(b) * a.sP +
                    static_cast<int64_t>(I) * kCB * a.ldp;
  const float* Qb = static_cast<const float*>(a.Q) + static_cast<int64_t>(b) * a.sQ +
                    static_cast<int64_t>(J) * kCB * a.ldq;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) acc[u][w] = 0.0;
  for (int k0 = 0; k0 < a.K; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * kCB; e += 256) {
      const int r = e >> 4, kk = e & 15;
      sP[kk][r] = Pb[static_cast<int64_t>(r) * a.ldp + k0 + kk];
      sQ[kk][r] = Qb[static_cast<int64_t>(r) * a.ldq + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      double p[4], q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = sP[kk][ty + 16 * u];
#pragma unroll
      for (int w = 0; w < 4; ++w) q[w] = sQ[kk][tx + 16 * w];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma(p[u], q[w], acc[u][w]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = I * kCB + ty + 16 * u;
      const int j = J * kCB + tx + 16 * w;
      if (a.sym && i < j) continue;
      epi_elem<kOpF32>(a, b, i, j, static_cast<float>(acc[u][w]), st);
    }
  block_partials<256>(a, b, blockIdx.x, red, st);
}

int gemm_tile(int op) { return op == kOpF32 ? kCB : kBM; }

hipError_t launch_gemm(const GemmArgs& a, int batch, int op, hipStream_t s) {
  dim3 grid(a.ntiles, batch), block(256);
  if (op == kOpBF16) {
    hipLaunchKernelGGL(gemm_nt_mfma<kOpBF16>, grid, block, 0, s, a);
  } else if (op == kOpF16) {
    hipLaunchKernelGGL(gemm_nt_mfma<kOpF16>, grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL(gemm_nt_f64acc, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace muon
