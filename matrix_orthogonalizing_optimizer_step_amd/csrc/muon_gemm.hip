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

// Epilogue, first half, for element (i, j) of matrix b (for symmetric
// products only i >= j is passed): v = alpha acc + beta E + gamma [i == j];
// stores v (and a fresh Q) at (i, j), accumulates the partial sums, and in
// the last product updates W (unless W is stored transposed, see epi_mirror).
template <int OP>
__device__ __forceinline__ float epi_value(const GemmArgs& a, int b, int i, int j, float acc, EpiState& st) {
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
    if (!a.transposed && i < a.n_real && j < a.m_real) {
      const int64_t idx = static_cast<int64_t>(i) * a.user_ld + j;
      if (a.W != nullptr) {
        void* w = a.W[b];
        const float wv = load_as_f32(w, idx, a.w_dtype);
        store_from_f32(w, idx, a.w_dtype, wv - a.lr * (v + a.wd * wv));
      }
      if (a.Oout != nullptr) store_from_f32(a.Oout[b], idx, a.o_dtype, v);
    }
    return v;
  }
  const int64_t o = static_cast<int64_t>(b) * a.sO + static_cast<int64_t>(i) * a.ldo + j;
  if (a.out32 != nullptr) a.out32[o] = v;
  if (a.out16 != nullptr) static_cast<T*>(a.out16)[o] = O::from_f(v);
  if (a.q32 != nullptr || a.q16 != nullptr) {
    const float q = diag ? v + st.ap : v;
    if (a.q32 != nullptr) a.q32[o] = q;
    if (a.q16 != nullptr) static_cast<T*>(a.q16)[o] = O::from_f(q);
  }
  if (a.part_out != nullptr && i < a.n_real && j < a.n_real) {
    if (diag) st.tr += v;
    st.ss += static_cast<double>(v) * v * ((a.sym && i != j) ? 2.0 : 1.0);
  }
  return v;
}

// Whether the transposed pass has work: mirrored symmetric stores, the X^T
// copy, or the update of a weight stored transposed.
__device__ __forceinline__ bool epi_has_mirror(const GemmArgs& a) {
  return a.final_mode ? a.transposed != 0 : (a.sym != 0 || a.outT16 != nullptr);
}

// Epilogue, second half: the stores at (j, i).
template <int OP>
__device__ __forceinline__ void epi_mirror(const GemmArgs& a, int b, int i, int j, float v, const EpiState& st) {
  using O = OpT<OP>;
  using T = typename O::T;
  if (a.final_mode) {
    if (i < a.n_real && j < a.m_real) {
      const int64_t idx = static_cast<int64_t>(j) * a.user_ld + i;
      if (a.W != nullptr) {
        void* w = a.W[b];
        const float wv = load_as_f32(w, idx, a.w_dtype);
        store_from_f32(w, idx, a.w_dtype, wv - a.lr * (v + a.wd * wv));
      }
      if (a.Oout != nullptr) store_from_f32(a.Oout[b], idx, a.o_dtype, v);
    }
    return;
  }
  if (a.sym) {
    if (i == j) return;
    const bool diag = false;
    const int64_t oT = static_cast<int64_t>(b) * a.sO + static_cast<int64_t>(j) * a.ldo + i;
    if (a.out32 != nullptr) a.out32[oT] = v;
    if (a.out16 != nullptr) static_cast<T*>(a.out16)[oT] = O::from_f(v);
    if (a.q32 != nullptr) a.q32[oT] = diag ? v + st.ap : v;
    if (a.q16 != nullptr) static_cast<T*>(a.q16)[oT] = O::from_f(v);
    return;
  }
  if (a.outT16 != nullptr) {
    static_cast<T*>(a.outT16)[static_cast<int64_t>(b) * a.sOT + static_cast<int64_t>(j) * a.ldot + i] =
        O::from_f(v);
  }
}

// ---------------------------------------------------------------------------
// Vectorised epilogue over a 32 x TN block of one wave's sub-tile, staged in
// LDS (row-major, leading dimension LDE floats).  Pass 1 gives each lane four
// consecutive columns of a row, batches the loads of several rows before any
// arithmetic, and stores at (i, j); pass 2 gives each lane four consecutive
// rows of a column for the stores at (j, i).
// ---------------------------------------------------------------------------
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

__device__ __forceinline__ float f4get(const float4& v, int k) {
  return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}
__device__ __forceinline__ void f4set(float4& v, int k, float x) {
  if (k == 0) v.x = x; else if (k == 1) v.y = x; else if (k == 2) v.z = x; else v.w = x;
}

// Four consecutive elements idx..idx+3 of a user buffer (dtype f32 or bf16):
// vector access when aligned and all four are in range, else element-wise.
__device__ __forceinline__ bool user4_vec(const void* p, int64_t idx, int dtype, int valid) {
  const int esz = dtype == kF32 ? 4 : 2;
  return valid >= 4 && ((reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(idx) * esz) & (4 * esz - 1)) == 0;
}
__device__ __forceinline__ float4 user_load4(const void* p, int64_t idx, int dtype, int valid) {
  if (user4_vec(p, idx, dtype, valid)) {
    if (dtype == kF32) return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
    const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + idx);
    return make_float4(bf16_to_f32(static_cast<uint16_t>(h.x & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(h.x >> 16)),
                       bf16_to_f32(static_cast<uint16_t>(h.y & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(h.y >> 16)));
  }
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < 4 && k < valid; ++k) f4set(r, k, load_as_f32(p, idx + k, dtype));
  return r;
}
__device__ __forceinline__ void user_store4(void* p, int64_t idx, int dtype, int valid, float4 v) {
  if (user4_vec(p, idx, dtype, valid)) {
    if (dtype == kF32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p) + idx) = v;
    } else {
      uint2 h;
      h.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
      h.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + idx) = h;
    }
    return;
  }
  for (int k = 0; k < 4 && k < valid; ++k) store_from_f32(p, idx + k, dtype, f4get(v, k));
}

// W <- W - lr (O + wd W) and the optional O store for four consecutive
// elements of the user's matrix at idx (valid of them in range).
__device__ __forceinline__ void final_update4(const GemmArgs& a, int b, int64_t idx, int valid, float4 o, float4 w) {
  if (valid <= 0) return;
  if (a.W != nullptr) {
    float4 nw;
    nw.x = w.x - a.lr * (o.x + a.wd * w.x);
    nw.y = w.y - a.lr * (o.y + a.wd * w.y);
    nw.z = w.z - a.lr * (o.z + a.wd * w.z);
    nw.w = w.w - a.lr * (o.w + a.wd * w.w);
    user_store4(a.W[b], idx, a.w_dtype, valid, nw);
  }
  if (a.Oout != nullptr) user_store4(a.Oout[b], idx, a.o_dtype, valid, o);
}

template <int OP, int TN, int LDE>
__device__ __forceinline__ void epilogue_block(const GemmArgs& a, int b, EpiState& st, float* ep, int i0, int j0,
                                               int lane, bool mirror) {
  using T = typename OpT<OP>::T;
  constexpr int LPR = TN / 4;        // lanes per row in pass 1
  constexpr int RPIT = 64 / LPR;     // rows per pass-1 iteration
  constexpr int NIT = 32 / RPIT;
  constexpr int UNR = NIT < 4 ? NIT : 4;
  const int cl = (lane % LPR) * 4;
  const int rl = lane / LPR;
  const bool has_e = a.E32 != nullptr || a.E16 != nullptr;
  const bool wrow = a.final_mode && !a.transposed && a.W != nullptr;
  for (int it0 = 0; it0 < NIT; it0 += UNR) {
    float4 ev[UNR], wv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + (it0 + u) * RPIT + rl, j = j0 + cl;
      ev[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      wv[u] = ev[u];
      const int64_t ie = static_cast<int64_t>(b) * a.sE + static_cast<int64_t>(i) * a.lde + j;
      if (has_e) ev[u] = a.E32 != nullptr ? load4_op<kOpF32>(a.E32, ie) : load4_op<OP>(a.E16, ie);
      if (wrow && i < a.n_real) {
        const int valid = a.m_real - j;
        if (valid > 0) wv[u] = user_load4(a.W[b], static_cast<int64_t>(i) * a.user_ld + j, a.w_dtype, valid);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int r = (it0 + u) * RPIT + rl;
      const int i = i0 + r, j = j0 + cl;
      float4* slot = reinterpret_cast<float4*>(ep + r * LDE + cl);
      const float4 acc = *slot;
      float4 v;
      v.x = st.alpha * acc.x + st.beta * ev[u].x;
      v.y = st.alpha * acc.y + st.beta * ev[u].y;
      v.z = st.alpha * acc.z + st.beta * ev[u].z;
      v.w = st.alpha * acc.w + st.beta * ev[u].w;
      const int dk = i - j;  // element k is on the diagonal when k == dk
      const bool dg = dk >= 0 && dk < 4 && i < a.n_real;
      if (dg) f4set(v, dk, f4get(v, dk) + st.gamma);
      *slot = v;
      if (a.final_mode) {
        if (!a.transposed && i < a.n_real) final_update4(a, b, static_cast<int64_t>(i) * a.user_ld + j, a.m_real - j, v, wv[u]);
        continue;
      }
      // symmetric products own i >= j only
      const int own = a.sym ? (dk >= 3 ? 4 : (dk < 0 ? 0 : dk + 1)) : 4;
      if (own == 0) continue;
      const int64_t o = static_cast<int64_t>(b) * a.sO + static_cast<int64_t>(i) * a.ldo + j;
      float4 q = v;
      if (dg) f4set(q, dk, f4get(q, dk) + st.ap);
      if (own == 4) {
        if (a.out32 != nullptr) store4_op<kOpF32>(a.out32, o, v);
        if (a.out16 != nullptr) store4_op<OP>(a.out16, o, v);
        if (a.q32 != nullptr) store4_op<kOpF32>(a.q32, o, q);
        if (a.q16 != nullptr) store4_op<OP>(a.q16, o, q);
      } else {
        for (int k = 0; k < own; ++k) {
          if (a.out32 != nullptr) a.out32[o + k] = f4get(v, k);
          if (a.out16 != nullptr) static_cast<T*>(a.out16)[o + k] = OpT<OP>::from_f(f4get(v, k));
          if (a.q32 != nullptr) a.q32[o + k] = f4get(q, k);
          if (a.q16 != nullptr) static_cast<T*>(a.q16)[o + k] = OpT<OP>::from_f(f4get(q, k));
        }
      }
      if (a.part_out != nullptr && i < a.n_real) {
        for (int k = 0; k < own; ++k) {
          if (j + k >= a.n_real) break;
          const double x = f4get(v, k);
          if (k == dk) st.tr += x;
          st.ss += x * x * ((a.sym && k != dk) ? 2.0 : 1.0);
        }
      }
    }
  }
  if (!mirror) return;
  __syncthreads();
  // pass 2: lane -> rows r4 .. r4 + 3 of column c
  const int r4 = (lane & 7) * 4;
  for (int c = lane >> 3; c < TN; c += 8) {
    const int i = i0 + r4, j = j0 + c;
    float4 v;
    v.x = ep[(r4 + 0) * LDE + c];
    v.y = ep[(r4 + 1) * LDE + c];
    v.z = ep[(r4 + 2) * LDE + c];
    v.w = ep[(r4 + 3) * LDE + c];
    if (a.final_mode) {  // weight stored transposed: W[j][i .. i + 3]
      if (j < a.m_real && i < a.n_real) {
        const int64_t idx = static_cast<int64_t>(j) * a.user_ld + i;
        const int valid = a.n_real - i;
        const float4 w = a.W != nullptr ? user_load4(a.W[b], idx, a.w_dtype, valid) : v;
        final_update4(a, b, idx, valid, v, w);
      }
      continue;
    }
    if (a.sym) {
      // elements i + k > j are mirrored to (j, i + k)
      const int first = j - i + 1;  // first k with i + k > j
      if (first >= 4) continue;
      const int64_t o = static_cast<int64_t>(b) * a.sO + static_cast<int64_t>(j) * a.ldo + i;
      if (first <= 0) {
        if (a.out32 != nullptr) store4_op<kOpF32>(a.out32, o, v);
        if (a.out16 != nullptr) store4_op<OP>(a.out16, o, v);
        if (a.q32 != nullptr) store4_op<kOpF32>(a.q32, o, v);
        if (a.q16 != nullptr) store4_op<OP>(a.q16, o, v);
      } else {
        for (int k = first; k < 4; ++k) {
          const float x = f4get(v, k);
          if (a.out32 != nullptr) a.out32[o + k] = x;
          if (a.out16 != nullptr) static_cast<T*>(a.out16)[o + k] = OpT<OP>::from_f(x);
          if (a.q32 != nullptr) a.q32[o + k] = x;
          if (a.q16 != nullptr) static_cast<T*>(a.q16)[o + k] = OpT<OP>::from_f(x);
        }
      }
    } else if (a.outT16 != nullptr) {
      store4_op<OP>(a.outT16, static_cast<int64_t>(b) * a.sOT + static_cast<int64_t>(j) * a.ldot + i, v);
    }
  }
}

// ---------------------------------------------------------------------------
// 16-bit MFMA kernel.  Block tile BM x BN, k-slab BK = 64, WGM x WGN waves,
// each wave owning a (BM/WGM) x (BN/WGN) sub-tile of 32x32x16 MFMA blocks.
// Operands are fetched with buffer loads (one descriptor per operand, the
// k offset in a scalar register) into registers one slab ahead, then stored
// to one of two LDS stages; 16-byte chunks are XOR-swizzled across rows so
// the fragment reads of 32 consecutive rows spread over all banks.
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

#ifndef MUON_BM
#define MUON_BM 256
#endif
#ifndef MUON_BN
#define MUON_BN 256
#endif
#ifndef MUON_WGM
#define MUON_WGM 2
#endif
#ifndef MUON_WGN
#define MUON_WGN 4
#endif
#ifndef MUON_BK
#define MUON_BK 32
#endif
#ifndef MUON_STAGES
#define MUON_STAGES 4
#endif

constexpr int kBM = MUON_BM, kBN = MUON_BN, kWGM = MUON_WGM, kWGN = MUON_WGN;
constexpr int kBK = MUON_BK, kCH = kBK / 8;  // k-slab and 16-byte chunks per slab row
constexpr int kStages = MUON_STAGES;
constexpr int kNT = 64 * kWGM * kWGN;
static_assert(kBK == 32 || kBK == 64, "k-slab of 32 or 64 elements");

// 16-byte chunk c of slab row r lives at chunk c ^ f(r) so that the
// fragment reads (32 consecutive rows, one chunk each) hit distinct banks
// for both 8- and 16-lane LDS service groups.
__device__ __forceinline__ int swz_f(int r) {
  return kCH == 8 ? ((r >> 1) & 7) : (((r >> 1) ^ (r >> 3)) & 3);
}
__device__ __forceinline__ int swz(int r, int c) { return r * kCH + (c ^ swz_f(r)); }

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4]
// (7 = no wait), lgkmcnt [11:8] (15 = no wait).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Copy one k-slab of ROWS rows from global memory straight into LDS.  One
// buffer_load ... lds instruction moves 1 KB: lane l lands at byte 16 l of the
// destination (rows r0 + l / kCH, physical chunk l % kCH), so the lane fetches
// the logical chunk the swizzle maps there.  PER_WAVE instructions per wave.
template <int ROWS>
__device__ __forceinline__ void slab_to_lds(__amdgpu_buffer_rsrc_t rsrc, const int* voff, int soff,
                                            uint4* stage_rows, int wave) {
  constexpr int RPI = 64 / kCH;                         // rows per instruction
  constexpr int PER_WAVE = ROWS / (kNT / 64) / RPI;
#pragma unroll
  for (int e = 0; e < PER_WAVE; ++e) {
    const int r0 = (wave * PER_WAVE + e) * RPI;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(stage_rows + r0 * kCH), 16, voff[e], soff, 0, 0);
  }
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int OP>
__global__ __launch_bounds__(kNT) void gemm_nt_mfma(GemmArgs a) {
  constexpr int TM = kBM / kWGM, TN = kBN / kWGN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int NW = kNT / 64;
  constexpr int RPI = 64 / kCH;
  constexpr int LP = kBM / NW / RPI, LQ = kBN / NW / RPI;  // direct-load instructions per wave per slab
  constexpr int STAGE = (kBM + kBN) * kCH;                 // uint4 per LDS stage
  constexpr int KS = kBK / 16;                             // MFMA k-steps per slab
  static_assert(FM <= 8, "the epilogue handles up to 8 MFMA rows per wave");
  static_assert(KS >= 2, "the barrier sits after the first k-step of a slab");
  __shared__ uint4 smem[kStages * STAGE];
  __shared__ double red[2 * kNT / 64];
  int b, tile, I, J;
  block_coords(a, kBM, kBN, b, tile, I, J);
  EpiState st;
  block_init<kNT>(a, b, tile, red, st);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t pbytes = (static_cast<int64_t>(a.Mdim - I * kBM) * a.ldp) * 2;
  const int64_t qbytes = (static_cast<int64_t>(a.Ndim - J * kBN) * a.ldq) * 2;
  const uint16_t* Pb = static_cast<const uint16_t*>(a.P) + static_cast<int64_t>(b) * a.sP +
                       static_cast<int64_t>(I) * kBM * a.ldp;
  const uint16_t* Qb = static_cast<const uint16_t*>(a.Q) + static_cast<int64_t>(b) * a.sQ +
                       static_cast<int64_t>(J) * kBN * a.ldq;
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(Pb, pbytes);
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Qb, qbytes);
  int voffP[LP], voffQ[LQ];
#pragma unroll
  for (int e = 0; e < LP; ++e) {
    const int r = (wave * LP + e) * RPI + lane / kCH;
    voffP[e] = (r * a.ldp + ((lane % kCH) ^ swz_f(r)) * 8) * 2;
  }
#pragma unroll
  for (int e = 0; e < LQ; ++e) {
    const int r = (wave * LQ + e) * RPI + lane / kCH;
    voffQ[e] = (r * a.ldq + ((lane % kCH) ^ swz_f(r)) * 8) * 2;
  }

  const int wm = wave / kWGN, wn = wave % kWGN;
  const int lr = lane & 31, lk = lane >> 5;
  int aoff[FM], boff[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) aoff[f] = wm * TM + f * 32 + lr;
#pragma unroll
  for (int f = 0; f < FN; ++f) boff[f] = kBM + wn * TN + f * 32 + lr;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int x = 0; x < FM; ++x)
#pragma unroll
    for (int y = 0; y < FN; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;

  const int nk = a.K / kBK;
  // prologue: slabs 0 .. kStages-1 in flight, one per stage
#pragma unroll
  for (int s0 = 0; s0 < kStages; ++s0) {
    if (s0 < nk) {
      slab_to_lds<kBM>(rP, voffP, s0 * kBK * 2, smem + s0 * STAGE, wave);
      slab_to_lds<kBN>(rQ, voffQ, s0 * kBK * 2, smem + s0 * STAGE + kBM * kCH, wave);
    }
  }
  // slab 0 landed for every wave
  if (nk >= kStages) __builtin_amdgcn_s_waitcnt(waitcnt_imm((kStages - 1) * (LP + LQ), 15));
  else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  block_barrier();

  uint4 af[2][FM], bf[2][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) af[0][f] = smem[swz(aoff[f], lk)];
#pragma unroll
  for (int f = 0; f < FN; ++f) bf[0][f] = smem[swz(boff[f], lk)];

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt % kStages) * STAGE;
    const int nxt = ((kt + 1) % kStages) * STAGE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int rb = ks & 1, wb = rb ^ 1;
      if (ks + 1 < KS) {
        const int c = (ks + 1) * 2 + lk;
#pragma unroll
        for (int f = 0; f < FM; ++f) af[wb][f] = smem[cur + swz(aoff[f], c)];
#pragma unroll
        for (int f = 0; f < FN; ++f) bf[wb][f] = smem[cur + swz(boff[f], c)];
      } else if (kt + 1 < nk) {
#pragma unroll
        for (int f = 0; f < FM; ++f) af[wb][f] = smem[nxt + swz(aoff[f], lk)];
#pragma unroll
        for (int f = 0; f < FN; ++f) bf[wb][f] = smem[nxt + swz(boff[f], lk)];
      }
#pragma unroll
      for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y) acc[x][y] = mfma32<OP>(af[rb][x], bf[rb][y], acc[x][y]);
#pragma unroll
      for (int g = 0; g < FM + FN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      if (ks == KS - 2) {
        // Every wave has read slab kt into registers and its own part of slab
        // kt + 1 has landed: after the barrier, slab kt + 1 is complete and
        // the stage of slab kt can take slab kt + kStages.  The MFMAs issued
        // above keep the matrix pipe busy while the wave waits here.
        if (kt + kStages - 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_imm((kStages - 2) * (LP + LQ), 0));
        else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kt + kStages < nk) {
          const int soff = (kt + kStages) * kBK * 2;
          slab_to_lds<kBM>(rP, voffP, soff, smem + cur, wave);
          slab_to_lds<kBN>(rQ, voffQ, soff, smem + cur + kBM * kCH, wave);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  block_barrier();

  // Epilogue: one 32-row block of every wave's sub-tile at a time is staged
  // through LDS (the MFMA 32x32 result layout: lane l, register v hold row
  // 8*(v/4) + 4*(l/32) + v%4, column l%32), then written out by
  // epilogue_block.
  constexpr int LDE = TN + 4;
  static_assert(kWGM * kWGN * 32 * LDE * 4 <= sizeof(smem), "epilogue staging must fit in LDS");
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * LDE;
  const bool mirror = epi_has_mirror(a);
  // The x loop stays rolled (its body is large); the accumulator row is
  // picked with constant indices so acc never needs dynamic indexing.
  for (int x = 0; x < FM; ++x) {
    switch (x) {
#define MUON_SCATTER_ROW(X)                                                                      \
  case X:                                                                                        \
    if constexpr (X < FM) {                                                                      \
      _Pragma("unroll") for (int y = 0; y < FN; ++y)                                             \
          _Pragma("unroll") for (int v = 0; v < 16; ++v)                                         \
              ep[(8 * (v >> 2) + 4 * lk + (v & 3)) * LDE + y * 32 + lr] = acc[X][y][v];           \
    }                                                                                            \
    break;
      MUON_SCATTER_ROW(0)
      MUON_SCATTER_ROW(1)
      MUON_SCATTER_ROW(2)
      MUON_SCATTER_ROW(3)
      MUON_SCATTER_ROW(4)
      MUON_SCATTER_ROW(5)
      MUON_SCATTER_ROW(6)
      MUON_SCATTER_ROW(7)
#undef MUON_SCATTER_ROW
      default:
        break;
    }
    __syncthreads();
    epilogue_block<OP, TN, LDE>(a, b, st, ep, I * kBM + wm * TM + x * 32, J * kBN + wn * TN, lane, mirror);
    __syncthreads();
  }
  block_partials<kNT>(a, b, tile, red, st);
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
  int b, tile, I, J;
  block_coords(a, kCB, kCB, b, tile, I, J);
  EpiState st;
  block_init<256>(a, b, tile, red, st);
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
      const float v = epi_value<kOpF32>(a, b, i, j, static_cast<float>(acc[u][w]), st);
      if (epi_has_mirror(a) && !(a.sym && i == j)) epi_mirror<kOpF32>(a, b, i, j, v, st);
    }
  block_partials<256>(a, b, tile, red, st);
}

int gemm_tile(int op) { return op == kOpF32 ? kCB : kBM; }

hipError_t launch_gemm(const GemmArgs& a, int batch, int op, hipStream_t s) {
  dim3 grid(a.ntiles, batch);
  if (op == kOpBF16) {
    hipLaunchKernelGGL(gemm_nt_mfma<kOpBF16>, grid, dim3(kNT), 0, s, a);
  } else if (op == kOpF16) {
    hipLaunchKernelGGL(gemm_nt_mfma<kOpF16>, grid, dim3(kNT), 0, s, a);
  } else {
    hipLaunchKernelGGL(gemm_nt_f64acc, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace muon
