// Batched GEMM kernels for the Newton-Schulz iterations, with fused epilogues.
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
__device__ __forceinline__ void final_update4(const GemmArgs& a, const EpiState& st, int64_t idx, int valid, float4 o,
                                              float4 w) {
  if (valid <= 0) return;
  if (st.w != nullptr) {
    float4 nw;
    nw.x = w.x - a.lr * (o.x + a.wd * w.x);
    nw.y = w.y - a.lr * (o.y + a.wd * w.y);
    nw.z = w.z - a.lr * (o.z + a.wd * w.z);
    nw.w = w.w - a.lr * (o.w + a.wd * w.w);
    user_store4(st.w, idx, a.w_dtype, valid, nw);
  }
  if (st.o != nullptr) user_store4(st.o, idx, a.o_dtype, valid, o);
}

// Epilogue over a 32 x TN block of C staged in LDS (row-major, leading
// dimension LDE floats), rows i0.., columns j0..  Pass 1 gives each lane four
// consecutive columns of a row (loads of several rows are issued before any
// arithmetic) and stores at (i, j); pass 2 gives each lane four consecutive
// rows of a column for the stores at (j, i).  All threads of the block call
// it (it contains a barrier).
template <int OP, int TN, int LDE>
__device__ __forceinline__ void epilogue_block(const GemmArgs& a, int b, EpiState& st, float* ep, int i0, int j0,
                                               int lane, bool mirror) {
  constexpr int LPR = TN / 4;        // lanes per row in pass 1
  constexpr int RPIT = 64 / LPR;     // rows per pass-1 iteration
  constexpr int NIT = 32 / RPIT;
  constexpr int UNR = NIT < 4 ? NIT : 4;
  const int cl = (lane % LPR) * 4;
  const int rl = lane / LPR;
  const bool has_e = a.E32 != nullptr || a.E16 != nullptr;
  const bool wrow = a.final_mode && !a.transposed && a.W != nullptr;
  const int64_t bE = static_cast<int64_t>(b) * a.sE;
  const int64_t bO = static_cast<int64_t>(b) * a.sO;
  for (int it0 = 0; it0 < NIT; it0 += UNR) {
    float4 ev[UNR], wv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + (it0 + u) * RPIT + rl, j = j0 + cl;
      ev[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      wv[u] = ev[u];
      if (a.E32 != nullptr) ev[u] = load4_op<kOpF32>(a.E32, bE + static_cast<int64_t>(i) * a.lde + j);
      else if (has_e) ev[u] = load4_op<OP>(a.E16, bE + op_index<OP>(i, j, a.lde));
      if (wrow && i < a.n_real) {
        const int valid = a.m_real - j;
        if (valid > 0) wv[u] = user_load4(st.w, static_cast<int64_t>(i) * a.user_ld + j, a.w_dtype, valid);
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
        if (!a.transposed && i < a.n_real) final_update4(a, st, static_cast<int64_t>(i) * a.user_ld + j, a.m_real - j, v, wv[u]);
        continue;
      }
      // symmetric products own i >= j only
      const int own = a.sym ? (dk >= 3 ? 4 : (dk < 0 ? 0 : dk + 1)) : 4;
      if (own == 0) continue;
      float4 q = v;
      if (dg) f4set(q, dk, f4get(q, dk) + st.ap);
      const int64_t o32 = bO + static_cast<int64_t>(i) * a.ldo + j;
      const int64_t o16 = bO + op_index<OP>(i, j, a.ldo);
      if (own == 4) {
        if (a.out32 != nullptr) store4_op<kOpF32>(a.out32, o32, v);
        if (a.out16 != nullptr) store4_op<OP>(a.out16, o16, v);
        if (a.q32 != nullptr) store4_op<kOpF32>(a.q32, o32, q);
        if (a.q16 != nullptr) store4_op<OP>(a.q16, o16, q);
      } else {
        for (int k = 0; k < own; ++k) {
          if (a.out32 != nullptr) a.out32[o32 + k] = f4get(v, k);
          if (a.out16 != nullptr) store1_op<OP>(a.out16, o16 + k, f4get(v, k));
          if (a.q32 != nullptr) a.q32[o32 + k] = f4get(q, k);
          if (a.q16 != nullptr) store1_op<OP>(a.q16, o16 + k, f4get(q, k));
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
        const float4 w = st.w != nullptr ? user_load4(st.w, idx, a.w_dtype, valid) : v;
        final_update4(a, st, idx, valid, v, w);
      }
      continue;
    }
    if (a.sym) {
      // elements i + k > j are mirrored to (j, i + k)
      const int first = j - i + 1;  // first k with i + k > j
      if (first >= 4) continue;
      const int64_t o32 = bO + static_cast<int64_t>(j) * a.ldo + i;
      const int64_t o16 = bO + op_index<OP>(j, i, a.ldo);
      if (first <= 0) {
        if (a.out32 != nullptr) store4_op<kOpF32>(a.out32, o32, v);
        if (a.out16 != nullptr) store4_op<OP>(a.out16, o16, v);
        if (a.q32 != nullptr) store4_op<kOpF32>(a.q32, o32, v);
        if (a.q16 != nullptr) store4_op<OP>(a.q16, o16, v);
      } else {
        for (int k = first; k < 4; ++k) {
          const float x = f4get(v, k);
          if (a.out32 != nullptr) a.out32[o32 + k] = x;
          if (a.out16 != nullptr) store1_op<OP>(a.out16, o16 + k, x);
          if (a.q32 != nullptr) a.q32[o32 + k] = x;
          if (a.q16 != nullptr) store1_op<OP>(a.q16, o16 + k, x);
        }
      }
    } else if (a.outT16 != nullptr) {
      store4_op<OP>(a.outT16, static_cast<int64_t>(b) * a.sOT + op_index<OP>(j, i, a.ldot), v);
    }
  }
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

// ---------------------------------------------------------------------------
// 16-bit MFMA kernel on packed operands.
//
// Block tile 256 (i) x 256 (j), 4 waves; wave w owns rows i0 + 64 w .. + 64
// against all 256 columns (2 x 8 MFMA 32x32x16 blocks, 256 accumulator
// registers).  k runs in slabs of 64 (4 MFMA k-steps):
//  * the P rows of a wave are private to it, so its P fragments go straight
//    from global memory (L2) into registers with one contiguous 1 KB load per
//    fragment, two slabs ahead (three register slab buffers);
//  * the Q tile is shared by all waves: it is streamed into a 4-stage LDS
//    ring with buffer_load ... lds (1 KB per instruction, lane l landing at
//    byte 16 l), three slabs ahead, and each fragment is read back with one
//    contiguous, conflict-free 16-byte-per-lane LDS read.
// One barrier per slab, after the third k-step: by then every wave has read
// the whole slab into registers, so its stage can take the slab four ahead,
// and the MFMAs already issued keep the matrix pipe busy through the wait.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kNW = 4, kNT = 64 * kNW;
constexpr int kFM = kBM / kNW / 32;   // MFMA row blocks per wave (2)
constexpr int kFN = kBN / 32;         // MFMA column blocks per wave (8)
constexpr int kKS = kBK / 16;         // k-steps per slab (4)
constexpr int kStages = 4;            // LDS ring depth for Q
constexpr int kStageBytes = kBN * kBK * 2;   // 32 KB
constexpr int kTN = kBN;              // epilogue: columns per wave
constexpr int kLDE = kTN + 4;         // staged row length (floats)
// each LDS stage array also holds one wave's 32-row epilogue staging block
constexpr int kStageAlloc = kStageBytes > 32 * kLDE * 4 ? kStageBytes : 32 * kLDE * 4;
// per-wave loads per slab: P: kFM row blocks x kKS fragments; Q: 8 row blocks / kNW waves x kKS
constexpr int kLoadsA = kFM * kKS;
constexpr int kLoadsB = (kBN / 32) / kNW * kKS;
static_assert(kLoadsA == kLoadsB, "the vmcnt bookkeeping assumes equal A and B load groups");

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4]
// (7 = no wait), lgkmcnt [11:8] (15 = no wait).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The P fragments of slab kt for this wave: kFM row blocks x kKS k-steps.
__device__ __forceinline__ void load_a_slab(uint4 (&buf)[kFM][kKS], __amdgpu_buffer_rsrc_t r, int voff,
                                            int sbase, int rb_stride, int kt) {
#pragma unroll
  for (int f = 0; f < kFM; ++f)
#pragma unroll
    for (int s = 0; s < kKS; ++s)
      buf[f][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                r, voff, sbase + f * rb_stride + kt * 4096 + s * 1024, 0));
}

// The Q slab kt into LDS stage `stage`: this wave's 2 row blocks x 4 fragments.
__device__ __forceinline__ void load_b_slab(uint4* stage, __amdgpu_buffer_rsrc_t r, int voff, int sbase,
                                            int rb_stride, int kt, int wave) {
#pragma unroll
  for (int f = 0; f < (kBN / 32) / kNW; ++f) {
    const int rb = wave * ((kBN / 32) / kNW) + f;
#pragma unroll
    for (int s = 0; s < kKS; ++s)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(stage + (rb * kKS + s) * 64), 16, voff,
                                               sbase + rb * rb_stride + kt * 4096 + s * 1024, 0, 0);
  }
}

// MFMAs of one k-step with the Q fragments of the next k-step read in between.
template <int OP>
__device__ __forceinline__ void kstep(f32x16_t (&acc)[kFM][kFN], const uint4 (&a)[kFM][kKS], int s,
                                      const uint4 (&bcur)[kFN], uint4 (&bnext)[kFN], const uint4* next_frags,
                                      bool read_next, int lane) {
  if (read_next) {
#pragma unroll
    for (int y = 0; y < kFN; ++y) bnext[y] = next_frags[y * kKS * 64 + lane];
  }
#pragma unroll
  for (int y = 0; y < kFN; ++y)
#pragma unroll
    for (int x = 0; x < kFM; ++x) acc[x][y] = mfma32<OP>(a[x][s], bcur[y], acc[x][y]);
  if (read_next) {
#pragma unroll
    for (int g = 0; g < kFN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    }
  }
}

// One slab: k-steps 0..3 of slab kt from registers `a` and LDS stage `cur`,
// reading ahead into bf; the barrier and the ring refill (slab kt + 4 into
// `cur`) sit after k-step 2.  Loads are issued unconditionally, also past
// the last slab: buffer loads are range-checked against the descriptor and
// the data is never used, and straight-line code lets the compiler count
// outstanding loads exactly.
template <int OP>
__device__ __forceinline__ void slab(f32x16_t (&acc)[kFM][kFN], const uint4 (&a)[kFM][kKS], uint4 (&bf)[2][kFN],
                                     uint4* cur, const uint4* nxt, __amdgpu_buffer_rsrc_t rQ, int voff, int sQ,
                                     int qstride, int kt, int wave, int lane) {
  kstep<OP>(acc, a, 0, bf[0], bf[1], cur + 1 * 64, true, lane);
  kstep<OP>(acc, a, 1, bf[1], bf[0], cur + 2 * 64, true, lane);
  kstep<OP>(acc, a, 2, bf[0], bf[1], cur + 3 * 64, true, lane);
  // This wave's reads of slab kt have landed and its part of slab kt + 1 is
  // in LDS (the 5 load groups issued after it may still be in flight); after
  // the barrier the whole slab kt + 1 is visible and nobody reads `cur`.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(5 * kLoadsB, 0));
  block_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_b_slab(cur, rQ, voff, sQ, qstride, kt + kStages, wave);
  kstep<OP>(acc, a, 3, bf[1], bf[0], nxt, true, lane);
}

// ---------------------------------------------------------------------------
// Register epilogue of the MFMA kernel.
//
// For the 32 x 32 MFMA block at rows ib.., columns jb.. a lane holds 16
// values in the accumulator arrangement "A": lane l, register r is element
//   (ib + 8 (r / 4) + 4 (l / 32) + r % 4,  jb + l % 32).
// Exchanging registers 4..7 of the lower half-wave with registers 0..3 of the
// upper half-wave (and 12..15 with 8..11) by v_permlane32_swap gives "N":
// lane l, register 8 h + e is (ib + 16 h + 8 (l / 32) + e, jb + l % 32), so a
// lane holds 8 consecutive rows of one column: in the packed operand layout
// that is this lane's 16 bytes of a fragment of C^T (row j, k = i).  Using
// such a fragment as the MFMA A operand against an identity B fragment gives
// the block transposed, exactly (products with 1 and sums with 0), in
// arrangement "T": lane l, register 8 h + e is (ib + l % 32, jb + 16 h +
// 8 (l / 32) + e), a fragment of C itself (row i, k = j).  Both C and C^T are
// thus written as whole 1 KB fragments from registers, and the 16-bit
// epilogue input is read as fragments of E^T (E is symmetric, or E = X read
// from X^T).
//
// fp32 side matrices (R, Q, RZ of the Gram iteration) are only ever read by
// this epilogue at the same block positions, so they are kept in arrangement
// A, one 4 KB record per 32 x 32 block (lower-triangle blocks only): record
// (ib / 32, jb / 32) of an ld x ld matrix, register r of lane l at offset
// 256 (r / 4) + 4 l + r % 4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t acc_rec(int ib, int jb, int ld) {
  return (static_cast<int64_t>(ib >> 5) * (ld >> 5) + (jb >> 5)) << 10;
}

// Exchange the upper half-wave of x with the lower half-wave of y.
__device__ __forceinline__ void xchg_halves(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

template <int OP>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return OP == kOpBF16 ? f32x2_to_bf16x2(lo, hi) : f32x2_to_f16x2(lo, hi);
}

// 16 values in arrangement A -> two 16-bit fragments in arrangement N.
template <int OP>
__device__ __forceinline__ void a_to_n16(const float (&v)[16], uint4 (&f)[2]) {
  uint32_t d[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k] = pack2<OP>(v[2 * k], v[2 * k + 1]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    xchg_halves(d[4 * h], d[4 * h + 2]);
    xchg_halves(d[4 * h + 1], d[4 * h + 3]);
  }
  f[0] = make_uint4(d[0], d[1], d[2], d[3]);
  f[1] = make_uint4(d[4], d[5], d[6], d[7]);
}

// Two 16-bit fragments in arrangement N -> 16 fp32 values in arrangement A.
template <int OP>
__device__ __forceinline__ void n16_to_a(const uint4& f0, const uint4& f1, float (&v)[16]) {
  uint32_t d[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    xchg_halves(d[4 * h], d[4 * h + 2]);
    xchg_halves(d[4 * h + 1], d[4 * h + 3]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[2 * k] = OpT<OP>::to_f(static_cast<uint16_t>(d[k] & 0xffffu));
    v[2 * k + 1] = OpT<OP>::to_f(static_cast<uint16_t>(d[k] >> 16));
  }
}

// B fragment h of the 32 x 32 identity: lane l holds B[k][n] for n = l % 32,
// k = 8 (l / 32) + e, equal to 1 where n == 16 h + k.
template <int OP>
__device__ __forceinline__ uint4 ident_frag(int h, int lane) {
  const uint32_t one = OP == kOpBF16 ? 0x3F80u : 0x3C00u;
  const int e = (lane & 31) - 16 * h - 8 * (lane >> 5);
  uint32_t d[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) d[k] = (e >= 0 && (e >> 1) == k) ? one << (16 * (e & 1)) : 0u;
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// Fragments in arrangement N -> the transposed block in arrangement T.
template <int OP>
__device__ __forceinline__ void transpose16(const uint4 (&n)[2], const uint4 (&id)[2], uint4 (&t)[2]) {
  f32x16_t d;
#pragma unroll
  for (int r = 0; r < 16; ++r) d[r] = 0.0f;
  d = mfma32<OP>(n[0], id[0], d);
  d = mfma32<OP>(n[1], id[1], d);
  float dv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) dv[r] = d[r];
  a_to_n16<OP>(dv, t);
}

// Diagonal block of a symmetric product: N and T fragments address the same
// elements (p, q) = (l % 32, 16 h + 8 (l / 32) + e); keep the owned value
// C[max][min], which is T where p >= q and N elsewhere.
__device__ __forceinline__ uint4 sym_select(const uint4& t, const uint4& n, int h, int lane) {
  const int p = lane & 31, q0 = 16 * h + 8 * (lane >> 5);
  const uint32_t tv[4] = {t.x, t.y, t.z, t.w}, nv[4] = {n.x, n.y, n.z, n.w};
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = (p >= q0 + 2 * k ? 0x0000ffffu : 0u) | (p >= q0 + 2 * k + 1 ? 0xffff0000u : 0u);
    r[k] = (tv[k] & m) | (nv[k] & ~m);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int OP>
__device__ __forceinline__ void store_frag(void* base, int64_t off, int lane, const uint4& f) {
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off + 8 * lane) = f;
}

// The 16-bit stores of one block: both triangles of a symmetric product, or
// X (from T) and X^T (from N) of a general one.
template <int OP>
__device__ __forceinline__ void store16(const GemmArgs& a, void* out, int64_t bO, const float (&v)[16], int ib, int jb,
                                        int lane, const uint4 (&id)[2]) {
  uint4 n16[2], t16[2];
  a_to_n16<OP>(v, n16);
  transpose16<OP>(n16, id, t16);
  uint16_t* o = static_cast<uint16_t*>(out) + bO;
  if (ib == jb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) store_frag<OP>(o, op_index<OP>(ib, jb + 16 * h, a.ldo), lane, sym_select(t16[h], n16[h], h, lane));
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      store_frag<OP>(o, op_index<OP>(ib, jb + 16 * h, a.ldo), lane, t16[h]);
      store_frag<OP>(o, op_index<OP>(jb, ib + 16 * h, a.ldo), lane, n16[h]);
    }
  }
}

// Epilogue of one 32 x 32 block (see the comment above): v = alpha C +
// beta E + gamma [i == j < n_real] in arrangement A, then its stores and
// partial sums.  `ein` holds the block's epilogue input as loaded (16-bit
// fragments of E^T in ein[0..1], or the fp32 record in ein[0..3]).  FINAL:
// v goes to the wave's LDS staging area `ep` (row-major, kLDE floats per row,
// this block at column ycol) for the update of W.
template <int OP, bool FINAL>
__device__ __forceinline__ void epi_block(const GemmArgs& a, int b, EpiState& st, const f32x16_t& c,
                                          const uint4 (&ein)[4], int ib, int jb, int lane, const uint4 (&id)[2],
                                          float* ep, int ycol) {
  const bool dblk = ib == jb;
  const int jr = lane & 31, ir0 = 4 * (lane >> 5);
  float e[16];
  if (a.E16 != nullptr) {
    n16_to_a<OP>(ein[0], ein[1], e);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint4& w = ein[r >> 2];
      const uint32_t u = (r & 3) == 0 ? w.x : ((r & 3) == 1 ? w.y : ((r & 3) == 2 ? w.z : w.w));
      e[r] = a.E32 != nullptr ? __uint_as_float(u) : 0.0f;
    }
  }
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = st.alpha * c[r] + st.beta * e[r];
  if (dblk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + ir0 + (r & 3);
      if (ir == jr && ib + ir < a.n_real) v[r] += st.gamma;
    }
  }
  if constexpr (FINAL) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + ir0 + (r & 3)) * kLDE + ycol + jr] = v[r];
    return;
  }
  const int64_t bO = static_cast<int64_t>(b) * a.sO;
  if (a.part_out != nullptr) {  // symmetric products: an off-diagonal value stands for two
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + ir0 + (r & 3);
      const double x = v[r];
      if (!dblk || ir > jr) {
        st.ss += 2.0 * x * x;
      } else if (ir == jr) {
        st.ss += x * x;
        st.tr += x;
      }
    }
  }
  if (a.out32 != nullptr) {
    float* o = a.out32 + bO + acc_rec(ib, jb, a.ldo) + 4 * lane;
#pragma unroll
    for (int g = 0; g < 4; ++g) *reinterpret_cast<float4*>(o + 256 * g) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
  }
  if (a.sym) {
    if (a.out16 != nullptr) store16<OP>(a, a.out16, bO, v, ib, jb, lane, id);
  } else {
    uint4 n16[2];
    a_to_n16<OP>(v, n16);
    if (a.outT16 != nullptr) {
      uint16_t* o = static_cast<uint16_t*>(a.outT16) + static_cast<int64_t>(b) * a.sOT;
#pragma unroll
      for (int h = 0; h < 2; ++h) store_frag<OP>(o, op_index<OP>(jb, ib + 16 * h, a.ldot), lane, n16[h]);
    }
    if (a.out16 != nullptr) {
      uint4 t16[2];
      transpose16<OP>(n16, id, t16);
      uint16_t* o = static_cast<uint16_t*>(a.out16) + bO;
#pragma unroll
      for (int h = 0; h < 2; ++h) store_frag<OP>(o, op_index<OP>(ib, jb + 16 * h, a.ldo), lane, t16[h]);
    }
  }
  if (a.q32 != nullptr || a.q16 != nullptr) {  // a fresh Q = v + a' I (symmetric products)
    float q[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + ir0 + (r & 3);
      q[r] = (dblk && ir == jr && ib + ir < a.n_real) ? v[r] + st.ap : v[r];
    }
    if (a.q32 != nullptr) {
      float* o = a.q32 + bO + acc_rec(ib, jb, a.ldo) + 4 * lane;
#pragma unroll
      for (int g = 0; g < 4; ++g) *reinterpret_cast<float4*>(o + 256 * g) = make_float4(q[4 * g], q[4 * g + 1], q[4 * g + 2], q[4 * g + 3]);
    }
    if (a.q16 != nullptr) store16<OP>(a, a.q16, bO, q, ib, jb, lane, id);
  }
}

// Final product: W <- W - lr (O + wd W) and the optional store of O, for
// rows i0 .. i0 + 31 and columns j0 .. j0 + 255 of O staged in LDS
// (row-major, LDE floats per row).  The loads of W for 16 rows (or columns)
// are issued together before any of them is used.
template <int LDE>
__device__ __forceinline__ void final_rows(const GemmArgs& a, const EpiState& st, const float* ep, int i0, int j0,
                                           int lane) {
  constexpr int R = 16;
  if (!a.transposed) {  // W is n x m: lane -> columns j .. j + 3 of every row
    const int j = j0 + 4 * lane;
    const int valid = a.m_real - j;
    for (int r0 = 0; r0 < 32; r0 += R) {
      float4 w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = i0 + r0 + r;
        w[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (st.w != nullptr && i < a.n_real && valid > 0)
          w[r] = user_load4(st.w, static_cast<int64_t>(i) * a.user_ld + j, a.w_dtype, valid);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = i0 + r0 + r;
        if (i < a.n_real)
          final_update4(a, st, static_cast<int64_t>(i) * a.user_ld + j, valid,
                        *reinterpret_cast<const float4*>(ep + (r0 + r) * LDE + 4 * lane), w[r]);
      }
    }
  } else {  // W is m x n: lane -> W[j][i .. i + 3] for 32 columns j of O
    const int r4 = (lane & 7) * 4;
    const int i = i0 + r4;
    const int valid = a.n_real - i;
    for (int c0 = 0; c0 < 256; c0 += 8 * R) {
      float4 w[R];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int j = j0 + c0 + 8 * t + (lane >> 3);
        w[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (st.w != nullptr && j < a.m_real && valid > 0)
          w[t] = user_load4(st.w, static_cast<int64_t>(j) * a.user_ld + i, a.w_dtype, valid);
      }
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int c = c0 + 8 * t + (lane >> 3);
        if (j0 + c < a.m_real) {
          const float4 o = make_float4(ep[(r4 + 0) * LDE + c], ep[(r4 + 1) * LDE + c], ep[(r4 + 2) * LDE + c],
                                       ep[(r4 + 3) * LDE + c]);
          final_update4(a, st, static_cast<int64_t>(j0 + c) * a.user_ld + i, valid, o, w[t]);
        }
      }
    }
  }
}

// Four MFMA blocks (row block X, column blocks Y0 .. Y0 + 3) of the register
// epilogue: their epilogue inputs are loaded together first.  The blocks are
// spelled out (not a loop) so the accumulators are always named statically.
template <int OP, bool FINAL, int X, int Y0>
__device__ __forceinline__ void epi_group(const GemmArgs& a, int b, EpiState& st, const f32x16_t (&acc)[kFM][kFN],
                                          int I, int J, int wave, int lane, const uint4 (&id)[2], float* ep) {
  constexpr int kEG = 4;
  const int64_t bE = static_cast<int64_t>(b) * a.sE;
  const int ib = I * kBM + wave * (kBM / kNW) + 32 * X;
  const int jb0 = J * kBN + 32 * Y0;
  uint4 ein[kEG][4];
#pragma unroll
  for (int u = 0; u < kEG; ++u) {
    const int jb = jb0 + 32 * u;
    if (a.sym && ib < jb) continue;  // the mirror of an owned block
    if (a.E16 != nullptr) {
      const uint16_t* E16 = static_cast<const uint16_t*>(a.E16) + bE;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ein[u][h] = *reinterpret_cast<const uint4*>(E16 + op_index<OP>(jb, ib + 16 * h, a.lde) + 8 * lane);
    } else if (a.E32 != nullptr) {
      const float* E32 = a.E32 + bE + acc_rec(ib, jb, a.lde) + 4 * lane;
#pragma unroll
      for (int g = 0; g < 4; ++g) ein[u][g] = *reinterpret_cast<const uint4*>(E32 + 256 * g);
    }
  }
  if (!(a.sym && ib < jb0 + 0)) epi_block<OP, FINAL>(a, b, st, acc[X][Y0 + 0], ein[0], ib, jb0 + 0, lane, id, ep, 32 * (Y0 + 0));
  if (!(a.sym && ib < jb0 + 32)) epi_block<OP, FINAL>(a, b, st, acc[X][Y0 + 1], ein[1], ib, jb0 + 32, lane, id, ep, 32 * (Y0 + 1));
  if (!(a.sym && ib < jb0 + 64)) epi_block<OP, FINAL>(a, b, st, acc[X][Y0 + 2], ein[2], ib, jb0 + 64, lane, id, ep, 32 * (Y0 + 2));
  if (!(a.sym && ib < jb0 + 96)) epi_block<OP, FINAL>(a, b, st, acc[X][Y0 + 3], ein[3], ib, jb0 + 96, lane, id, ep, 32 * (Y0 + 3));
}

// The register epilogue over a wave's 64 x 256 sub-tile.
template <int OP>
__device__ __forceinline__ void epilogue_regs(const GemmArgs& a, int b, EpiState& st, const f32x16_t (&acc)[kFM][kFN],
                                              int I, int J, int wave, int lane) {
  static_assert(kFM == 2 && kFN == 8, "the epilogue groups are spelled out for 2 x 8 MFMA blocks");
  const uint4 id[2] = {ident_frag<OP>(0, lane), ident_frag<OP>(1, lane)};
  epi_group<OP, false, 0, 0>(a, b, st, acc, I, J, wave, lane, id, nullptr);
  epi_group<OP, false, 0, 4>(a, b, st, acc, I, J, wave, lane, id, nullptr);
  epi_group<OP, false, 1, 0>(a, b, st, acc, I, J, wave, lane, id, nullptr);
  epi_group<OP, false, 1, 4>(a, b, st, acc, I, J, wave, lane, id, nullptr);
}

// Final product, row block X of the wave: O = v goes through the wave's LDS
// staging area (row-major, kLDE floats per row) into the update of W, so the
// user's row-major W is read and written along its rows.
template <int OP, int X>
__device__ __forceinline__ void final_stage(const GemmArgs& a, int b, EpiState& st, const f32x16_t (&acc)[kFM][kFN],
                                            float* ep, int I, int J, int wave, int lane) {
  const uint4 id[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};  // unused in the final product
  epi_group<OP, true, X, 0>(a, b, st, acc, I, J, wave, lane, id, ep);
  epi_group<OP, true, X, 4>(a, b, st, acc, I, J, wave, lane, id, ep);
  __syncthreads();
  final_rows<kLDE>(a, st, ep, I * kBM + wave * (kBM / kNW) + X * 32, J * kBN, lane);
  __syncthreads();
}

template <int OP>
__global__ __launch_bounds__(kNT) void gemm_nt_mfma(GemmArgs a) {
  // The Q ring is four separate arrays, each named statically at every access,
  // so the compiler's wait for an LDS read covers only the DMA into that stage.
  __shared__ uint4 stg0[kStageAlloc / 16], stg1[kStageAlloc / 16], stg2[kStageAlloc / 16], stg3[kStageAlloc / 16];
  __shared__ double red[2 * kNW];
  int b, tile, I, J;
  block_coords(a, kBM, kBN, b, tile, I, J);
  EpiState st;
  block_init<kNT>(a, b, tile, red, st);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* Pm = static_cast<const uint16_t*>(a.P) + static_cast<int64_t>(b) * a.sP;
  const uint16_t* Qm = static_cast<const uint16_t*>(a.Q) + static_cast<int64_t>(b) * a.sQ;
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(Pm, static_cast<int64_t>(a.Mdim) * a.ldp * 2);
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Qm, static_cast<int64_t>(a.Ndim) * a.ldq * 2);
  const int voff = lane * 16;
  // byte offset of a row block = (row / 32) * (K / 64) * 4 KB
  const int pstride = (a.ldp >> 6) * 4096, qstride = (a.ldq >> 6) * 4096;
  const int sP = (I * (kBM / 32) + wave * kFM) * pstride;
  const int sQ = J * (kBN / 32) * qstride;

  f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int x = 0; x < kFM; ++x)
#pragma unroll
    for (int y = 0; y < kFN; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;

  const int nk = a.K / kBK;  // a multiple of 4: every operand dimension is a multiple of 256
  uint4 abuf0[kFM][kKS], abuf1[kFM][kKS], abuf2[kFM][kKS];
  uint4 bf[2][kFN];
  // prologue: Q slabs 0..3 into the ring, P slabs 0 and 1 into registers
  load_b_slab(stg0, rQ, voff, sQ, qstride, 0, wave);
  load_b_slab(stg1, rQ, voff, sQ, qstride, 1, wave);
  load_b_slab(stg2, rQ, voff, sQ, qstride, 2, wave);
  load_b_slab(stg3, rQ, voff, sQ, qstride, 3, wave);
  load_a_slab(abuf0, rP, voff, sP, pstride, 0);
  load_a_slab(abuf1, rP, voff, sP, pstride, 1);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(5 * kLoadsB, 15));  // Q slab 0 landed
  block_barrier();
#pragma unroll
  for (int y = 0; y < kFN; ++y) bf[0][y] = stg0[y * kKS * 64 + lane];

  // 12 slabs per trip (lcm of the 4 LDS stages and the 3 P register buffers);
  // nk is a multiple of 4, so a remainder of 4 or 8 slabs follows.
#define MUON_SLAB(U, BUF, NEXTBUF, CUR, NXT)                                                           \
  load_a_slab(NEXTBUF, rP, voff, sP, pstride, kt + U + 2);                                             \
  slab<OP>(acc, BUF, bf, CUR, NXT, rQ, voff, sQ, qstride, kt + U, wave, lane);
  int kt = 0;
  for (; kt + 12 <= nk; kt += 12) {
    MUON_SLAB(0, abuf0, abuf2, stg0, stg1)
    MUON_SLAB(1, abuf1, abuf0, stg1, stg2)
    MUON_SLAB(2, abuf2, abuf1, stg2, stg3)
    MUON_SLAB(3, abuf0, abuf2, stg3, stg0)
    MUON_SLAB(4, abuf1, abuf0, stg0, stg1)
    MUON_SLAB(5, abuf2, abuf1, stg1, stg2)
    MUON_SLAB(6, abuf0, abuf2, stg2, stg3)
    MUON_SLAB(7, abuf1, abuf0, stg3, stg0)
    MUON_SLAB(8, abuf2, abuf1, stg0, stg1)
    MUON_SLAB(9, abuf0, abuf2, stg1, stg2)
    MUON_SLAB(10, abuf1, abuf0, stg2, stg3)
    MUON_SLAB(11, abuf2, abuf1, stg3, stg0)
  }
  if (kt + 4 <= nk) {
    MUON_SLAB(0, abuf0, abuf2, stg0, stg1)
    MUON_SLAB(1, abuf1, abuf0, stg1, stg2)
    MUON_SLAB(2, abuf2, abuf1, stg2, stg3)
    MUON_SLAB(3, abuf0, abuf2, stg3, stg0)
    if (kt + 8 <= nk) {
      MUON_SLAB(4, abuf1, abuf0, stg0, stg1)
      MUON_SLAB(5, abuf2, abuf1, stg1, stg2)
      MUON_SLAB(6, abuf0, abuf2, stg2, stg3)
      MUON_SLAB(7, abuf1, abuf0, stg3, stg0)
    }
  }
#undef MUON_SLAB
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  block_barrier();

  // Epilogue from registers; the final product goes through LDS.
  if (a.final_mode) {
    float* ep = reinterpret_cast<float*>(wave == 0 ? stg0 : (wave == 1 ? stg1 : (wave == 2 ? stg2 : stg3)));
    final_stage<OP, 0>(a, b, st, acc, ep, I, J, wave, lane);
    final_stage<OP, 1>(a, b, st, acc, ep, I, J, wave, lane);
  } else {
    epilogue_regs<OP>(a, b, st, acc, I, J, wave, lane);
  }
  block_partials<kNT>(a, b, tile, red, st);
}

// ---------------------------------------------------------------------------
// fp32 check path: fp32 row-major operands, exact products and fp64
// accumulation.  64 x 64 block tile, 16 x 16 threads with 4 x 4 outputs each;
// the tile is staged in LDS and written by the same epilogue.  Slow.
// ---------------------------------------------------------------------------
constexpr int kCB = 64;

__global__ __launch_bounds__(256) void gemm_nt_f64acc(GemmArgs a) {
  __shared__ float sP[16][kCB + 1];
  __shared__ float sQ[16][kCB + 1];
  __shared__ float stage[4][32 * (32 + 4)];
  __shared__ double red[8];
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
  // 64 x 64 tile = 2 x 2 blocks of 32 x 32, one per wave
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* ep = stage[wave];
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int r = ty + 16 * u, c = tx + 16 * w;  // position in the 64 x 64 tile
      stage[(r >> 5) * 2 + (c >> 5)][(r & 31) * 36 + (c & 31)] = static_cast<float>(acc[u][w]);
    }
  __syncthreads();
  epilogue_block<kOpF32, 32, 36>(a, b, st, ep, I * kCB + wr, J * kCB + wc, lane, epi_has_mirror(a));
  __syncthreads();
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
