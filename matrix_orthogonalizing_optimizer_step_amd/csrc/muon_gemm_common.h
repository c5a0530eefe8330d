// Batched GEMM kernels for the Newton-Schulz iterations, with fused epilogues:
// the parts shared by the MFMA kernels and the fp32 check path.
//
// Every product of the standard and Gram Newton-Schulz iterations ([GNS §1.2]
// and [GNS §2.3-3.4] of the Gram Newton-Schulz notes) is written in the
// "NT" form C[i][j] = sum_k P[i][k] Q[j][k] over k:
//   X X^T            P = Q = X (n x m)                      symmetric
//   A A, R R, Q Z,   P, Q symmetric n x n (Q^T = Q)         symmetric
//   R Z, Z (RZ)
//   B X, Q X         P = B or Q (n x n), Q = X^T (m x n)    general
// X is kept in both layouts (X and X^T) by the producing epilogue, so one
// tile loop serves every product.  Symmetric products compute only the tiles
// on or below the diagonal and store each value at (i, j) and (j, i), the
// triangle-only scheme the notes describe for their symmetric GEMM [GNS §4].
//
// 16-bit operands are stored in a packed fragment layout (op_index below):
// each 32-row x 16-k block is 1 KB in the lane order of the MFMA operand, so
// a wave fetches a fragment with one contiguous 16-byte-per-lane access,
// from global memory or from LDS.  They run on CDNA4 MFMA
// (v_mfma_f32_32x32x16_{bf16,f16}) with fp32 accumulation.  The fp32 check
// path keeps row-major fp32 operands and accumulates in fp64.
#pragma once

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
  void* w;  // this matrix's W and O in the final product (read once, before any store)
  void* o;
};

// The diagonal shift a' of matrix b: mean of a + b l + c l^2 over the
// eigenvalues l of the Gram matrix, from its trace and Frobenius norm (both
// reduced from per-tile partials in a fixed order, so every block of a
// launch gets the same value).  All threads of the block must call this.
template <int NT>
__device__ __forceinline__ float block_shift(const GemmArgs& a, int b, double* red) {
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
__device__ __forceinline__ void block_init(const GemmArgs& a, int b, int tile, double* red, EpiState& st) {
  st.ap = block_shift<NT>(a, b, red);
  if (a.shift_out != nullptr && tile == 0 && threadIdx.x == 0) a.shift_out[b] = st.ap;
  st.alpha = a.alpha_c + a.alpha_a * st.ap;
  st.beta = a.beta_c + a.beta_a * st.ap;
  st.gamma = a.gamma_c + a.gamma_a * st.ap;
  st.tr = 0.0;
  st.ss = 0.0;
  st.w = a.final_mode && a.W != nullptr ? a.W[b] : nullptr;
  st.o = a.final_mode && a.Oout != nullptr ? a.Oout[b] : nullptr;
}

// Write the (trace, sum of squares) partial of this tile.
template <int NT>
__device__ __forceinline__ void block_partials(const GemmArgs& a, int b, int tile, double* red, EpiState& st) {
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

// ---------------------------------------------------------------------------
// Epilogue helpers.  The staged epilogue computes, per element of C,
//   v = alpha * C + beta * E[i][j] + gamma * [i == j < n_real]
// (alpha, beta, gamma affine in the diagonal shift a'), stores v in fp32
// and/or the 16-bit operand layout, a fresh Q = v + a' I, the per-tile trace
// and sum of squares, the transposed copy X^T, and in the last product the
// update of W.  For symmetric products a block owns the elements with i >= j
// and mirrors them to (j, i).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool epi_has_mirror(const GemmArgs& a) {
  return a.final_mode ? a.transposed != 0 : (a.sym != 0 || a.outT16 != nullptr);
}

template <int OP>
__device__ __forceinline__ float4 load4_op(const void* base, int64_t idx) {
  if constexpr (OP == kOpF32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  } else {
    const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return make_float4(OpT<OP>::to_f(static_cast<uint16_t>(h.x & 0xffffu)), OpT<OP>::to_f(static_cast<uint16_t>(h.x >> 16)),
                       OpT<OP>::to_f(static_cast<uint16_t>(h.y & 0xffffu)), OpT<OP>::to_f(static_cast<uint16_t>(h.y >> 16)));
  }
}

template <int OP>
__device__ __forceinline__ void store4_op(void* base, int64_t idx, float4 v) {
  if constexpr (OP == kOpF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = v;
  } else {
    using O = OpT<OP>;
    uint2 h;
    h.x = static_cast<uint32_t>(O::from_f(v.x)) | (static_cast<uint32_t>(O::from_f(v.y)) << 16);
    h.y = static_cast<uint32_t>(O::from_f(v.z)) | (static_cast<uint32_t>(O::from_f(v.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = h;
  }
}

template <int OP>
__device__ __forceinline__ void store1_op(void* base, int64_t idx, float v) {
  if constexpr (OP == kOpF32) {
    static_cast<float*>(base)[idx] = v;
  } else {
    static_cast<uint16_t*>(base)[idx] = OpT<OP>::from_f(v);
  }
}

__device__ __forceinline__ float f4get(const float4& v, int k) {
  return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}
__device__ __forceinline__ void f4set(float4& v, int k, float x) {
  if (k == 0) v.x = x; else if (k == 1) v.y = x; else if (k == 2) v.z = x; else v.w = x;
}

// Four consecutive elements idx..idx+3 of a user buffer (dtype f32 or bf16):
// vector access when aligned and all four are in range, else element-wise.
// The user's W and O are device memory: accessing them through
// global-address-space pointers gives global_* instead of flat_* instructions.
typedef float gf32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t gu32x2_t __attribute__((ext_vector_type(2)));
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gptr(void* p, int64_t idx) {
  return (__attribute__((address_space(1))) T*)p + idx;
}
__device__ __forceinline__ float4 gload_f32x4(void* p, int64_t byte_off) {
  const gf32x4_t v = *(__attribute__((address_space(1))) gf32x4_t*)gptr<char>(p, byte_off);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 gload_bf16x4(void* p, int64_t byte_off) {
  const gu32x2_t h = *(__attribute__((address_space(1))) gu32x2_t*)gptr<char>(p, byte_off);
  return make_float4(bf16_to_f32(static_cast<uint16_t>(h.x & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(h.x >> 16)),
                     bf16_to_f32(static_cast<uint16_t>(h.y & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(h.y >> 16)));
}
__device__ __forceinline__ void gstore_f32x4(void* p, int64_t byte_off, const float4& v) {
  *(__attribute__((address_space(1))) gf32x4_t*)gptr<char>(p, byte_off) = gf32x4_t{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void gstore_bf16x4(void* p, int64_t byte_off, const float4& v) {
  *(__attribute__((address_space(1))) gu32x2_t*)gptr<char>(p, byte_off) =
      gu32x2_t{f32x2_to_bf16x2(v.x, v.y), f32x2_to_bf16x2(v.z, v.w)};
}

__device__ __forceinline__ bool user4_vec(const void* p, int64_t idx, int dtype, int valid) {
  const int esz = dtype == kF32 ? 4 : 2;
  return valid >= 4 && ((reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(idx) * esz) & (4 * esz - 1)) == 0;
}
__device__ __forceinline__ float user_load1(void* p, int64_t idx, int dtype) {
  return dtype == kF32 ? *gptr<float>(p, idx) : bf16_to_f32(*gptr<uint16_t>(p, idx));
}
__device__ __forceinline__ void user_store1(void* p, int64_t idx, int dtype, float v) {
  if (dtype == kF32) {
    *gptr<float>(p, idx) = v;
  } else {
    *gptr<uint16_t>(p, idx) = f32_to_bf16(v);
  }
}
// Four consecutive elements idx .. idx + 3 of a user buffer (dtype f32 or
// bf16): vector access when aligned and all four are in range, else
// element-wise.
__device__ __forceinline__ float4 user_load4(void* p, int64_t idx, int dtype, int valid) {
  if (user4_vec(p, idx, dtype, valid)) return dtype == kF32 ? gload_f32x4(p, idx * 4) : gload_bf16x4(p, idx * 2);
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < 4 && k < valid; ++k) f4set(r, k, user_load1(p, idx + k, dtype));
  return r;
}
__device__ __forceinline__ void user_store4(void* p, int64_t idx, int dtype, int valid, float4 v) {
  if (user4_vec(p, idx, dtype, valid)) {
    if (dtype == kF32) {
      gstore_f32x4(p, idx * 4, v);
    } else {
      gstore_bf16x4(p, idx * 2, v);
    }
    return;
  }
  for (int k = 0; k < 4 && k < valid; ++k) user_store1(p, idx + k, dtype, f4get(v, k));
}

// W <- W - lr (s O + wd W) and the optional O store (O, unscaled) for four consecutive
// elements of the user's matrix at idx (valid of them in range).
__device__ __forceinline__ void final_update4(const GemmArgs& a, const EpiState& st, int64_t idx, int valid, float4 o,
                                              float4 w) {
  if (valid <= 0) return;
  if (st.w != nullptr) {
    float4 nw;
    nw.x = w.x - a.lr * (a.oscale * o.x + a.wd * w.x);
    nw.y = w.y - a.lr * (a.oscale * o.y + a.wd * w.y);
    nw.z = w.z - a.lr * (a.oscale * o.z + a.wd * w.z);
    nw.w = w.w - a.lr * (a.oscale * o.w + a.wd * w.w);
    user_store4(st.w, idx, a.w_dtype, valid, nw);
  }
  if (st.o != nullptr) user_store4(st.o, idx, a.o_dtype, valid, o);
}

// Map the linear block id to (matrix, tile): consecutive ids go to different
// XCDs (round-robin dispatch), so renumber such that each XCD works through a
// contiguous range of tiles, then order the tiles of a general product in
// groups of 8 tile-rows for L2 reuse of both operands.
__device__ __forceinline__ void block_coords(const GemmArgs& a, int BM, int BN, int& b, int& tile, int& I, int& J) {
  const int nb = a.ntiles * gridDim.y;
  int lin = blockIdx.y * a.ntiles + blockIdx.x;
  {
    // XCD x (= lin % 8) takes the x-th contiguous range of q or q + 1 tiles
    const int q = nb >> 3, rem = nb & 7, x = lin & 7, slot = lin >> 3;
    lin = (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + slot;
  }
  b = lin / a.ntiles;
  tile = lin - b * a.ntiles;
  if (a.sym) {
    tri_tile(tile, I, J);
  } else {
    const int ntm = a.Mdim / BM, ntn = a.Ndim / BN;
    constexpr int G = 8;
    const int grp = tile / (G * ntn);
    const int first = grp * G;
    const int rows = ntm - first < G ? ntm - first : G;
    const int in = tile - grp * G * ntn;
    I = first + in % rows;
    J = in / rows;
  }
}

}  // namespace muon
