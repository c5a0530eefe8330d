// fp32 check path of the GEMM: fp32 row-major operands, exact products and
// fp64 accumulation, with the epilogue staged through LDS in row-major order.
#include "muon_gemm_common.h"

namespace muon {

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
  const bool has_e = a.E16 != nullptr;
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
      if (has_e) ev[u] = load4_op<OP>(a.E16, bE + op_index<OP>(i, j, a.lde));
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
      const int64_t o16 = bO + op_index<OP>(i, j, a.ldo);
      if (own == 4) {
        if (a.out16 != nullptr) store4_op<OP>(a.out16, o16, v);
        if (a.q16 != nullptr) store4_op<OP>(a.q16, o16, q);
      } else {
        for (int k = 0; k < own; ++k) {
          if (a.out16 != nullptr) store1_op<OP>(a.out16, o16 + k, f4get(v, k));
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
      const int64_t o16 = bO + op_index<OP>(j, i, a.ldo);
      if (first <= 0) {
        if (a.out16 != nullptr) store4_op<OP>(a.out16, o16, v);
        if (a.q16 != nullptr) store4_op<OP>(a.q16, o16, v);
      } else {
        for (int k = first; k < 4; ++k) {
          const float x = f4get(v, k);
          if (a.out16 != nullptr) store1_op<OP>(a.out16, o16 + k, x);
          if (a.q16 != nullptr) store1_op<OP>(a.q16, o16 + k, x);
        }
      }
    } else if (a.outT16 != nullptr) {
      store4_op<OP>(a.outT16, static_cast<int64_t>(b) * a.sOT + op_index<OP>(j, i, a.ldot), v);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 check path: fp32 row-major operands, exact products and fp64
// accumulation.  64 x 64 block tile, 16 x 16 threads with 4 x 4 outputs each;
// the tile is staged in LDS and written by the same epilogue.  Slow.
// ---------------------------------------------------------------------------
constexpr int kCB = kCheckTile;

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

hipError_t launch_gemm_f32(const GemmArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(gemm_nt_f64acc, dim3(a.ntiles, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
