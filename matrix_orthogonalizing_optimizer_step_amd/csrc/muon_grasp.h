// Internal declarations of the low-bit momentum state kernels (muon_grasp.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

constexpr int kGridBlock = 128;  // grid block edge and 8-bit group length

// 4-bit grid code over 128 x 128 blocks; matrix arguments are device arrays of
// per-matrix device pointers, except the fp32 M_t buffer (strided).
struct GridArgs {
  int rows, cols;
  const void* const* X;                         // mode 0: fp32 input
  void* const* codes;                           // uint8 rows x (cols + 1) / 2
  void* const* sr;                              // fp32 rows x ceil(cols / 128)
  void* const* sc;                              // fp32 ceil(rows / 128) x cols
  const void* const* G; int g_dtype; double mu; // mode 1
  void* const* Y;                               // mode 1: optional copy of M_t; mode 2: output
  float* mt; int64_t s_mt;                      // mode 1: M_t of matrix b at mt + b * s_mt
};

// 8-bit groups of 128 along the rows of a rows x k matrix.
struct Group8Args {
  int rows, k;
  void* const* Xp; float* Xs; int64_t sX;       // fp32 values: pointer array, or strided if Xp is null
  void* const* codes;                           // int8 rows x k
  void* const* scales;                          // fp32 rows x ceil(k / 128)
};

// Column norms of the decoded R_{t-1} (n x k).
constexpr int kUnitRows = 64;  // rows per chunk of the column sums
struct UnitArgs {
  int n, k, nchunk;                             // nchunk = ceil(n / kUnitRows)
  const void* const* codes; const void* const* scales;
  double* part;                                 // batch x nchunk x k
  double* inv;                                  // batch x k: 1 / column norm
};

// P~ = M_t Q with Q the unit columns of deq(R_{t-1}) (rows x cols times cols x
// k): Q[j][c] = q_jc s_{j,c/128} inv_c / 127, so the column tile of 128
// columns c (one 8-bit group g) is (inv_c / 127) sum_j (M_t[i][j] s_{j,g})
// q_jc, with the codes exact in bf16.  With pieces > 1 as TallArgs.
struct MQArgs {
  int M, N, K;                                  // rows, k, cols
  const float* A; int64_t sA;                   // M_t, matrix b at A + b sA
  const uint16_t* Ct; int64_t sCt;              // R's codes transposed, bf16 (k x cols), matrix b at + b sCt
  const void* const* rs;                        // R's group scales (cols x ceil(k / 128)) per matrix
  const double* inv;                            // batch x k: 1 / column norm of deq(R_{t-1})
  float* C; int64_t sC;
  int pieces, kchunk;
};

// C[b] (M x N, row-major, fp32) = A[b] B[b]; A element (row, k) at
// A + b sA + row a_row + k a_k, B element (col, k) at B + b sB + col b_row + k b_k.
// With pieces > 1, block z = b * pieces + p covers k in [p kchunk, (p + 1) kchunk)
// and writes C + z sC (partial products, summed by launch_sum_pieces).
// Bh / Bl non-null: B comes pre-split into bf16 planes (hi, lo), element
// (col, k) at + b sB + col b_row + k (k contiguous); B and b_k are unused.
// Ah / Al likewise for A (element (row, k) at + b sA + row a_row + k), taken
// by the residual kernel only.
struct TallArgs {
  int M, N, K;
  const float* A; int64_t sA, a_row, a_k;
  const float* B; int64_t sB, b_row, b_k;
  float* C; int64_t sC;
  int pieces, kchunk;
  const uint16_t* Bh = nullptr;
  const uint16_t* Bl = nullptr;
  const uint16_t* Ah = nullptr;
  const uint16_t* Al = nullptr;
};

// M_t = mu (deq(M_res) + deq(P) deq(R)^T) + G.
struct ReconArgs {
  int rows, cols, k;
  const void* const* res_codes; const void* const* res_sr; const void* const* res_sc;
  const void* const* P_codes; const void* const* P_scales;
  const void* const* R_codes; const void* const* R_scales;
  const void* const* G; int g_dtype; double mu;
  float* mt; int64_t s_mt;
  void* const* Y;                               // optional copy of M_t
};

// New grid code of M_t - P R^T (prod: A = P, B = R, both pre-split into bf16
// planes, k contiguous).
struct ResidualArgs {
  int rows, cols;
  TallArgs prod;
  const float* mt; int64_t s_mt;
  void* const* codes; void* const* sr; void* const* sc;
};

// CholeskyQR of P~ (m x k): partial Gram matrices, their sum S, the factor U
// (in place of S) and P = P~ U^{-1}.
struct CholArgs {
  int m, k, nchunk, chunk;                      // Gram partials over chunks of `chunk` rows
  const float* P; int64_t sP;                   // P~ (input)
  double* spart;                                // batch x nchunk x k x k
  double* S;                                    // batch x k x k (becomes U)
  int* dead;                                    // batch x k: 1 for a dependent or zero column
  float* Pout;                                  // P (m x k, same strides as P~)
  int panel;                                    // Cholesky panel rows (set by the launcher)
  double* dinv;                                 // batch x ceil(k / 64) x 64 x 64: U's diagonal blocks inverted
};

// Largest subspace rank of the register-resident Cholesky; larger ranks take
// the panel kernel.
constexpr int kRegRankK = 256;

// Largest subspace rank the kernels take.
constexpr int kMaxRankK = 1024;

// Rows per Gram partial: 64, or more when the batch alone gives ~1024 blocks.
inline int gram_chunk_rows(int m, int batch) {
  const int64_t per = (static_cast<int64_t>(m) * batch + 1023) / 1024;
  return static_cast<int>((per + 63) / 64 * 64);
}

hipError_t launch_grid(const GridArgs& a, int mode, int batch, hipStream_t s);
hipError_t launch_group8(const Group8Args& a, bool dequantize, int batch, hipStream_t s);
hipError_t launch_col_norms(const UnitArgs& a, int batch, hipStream_t s);
hipError_t launch_codes_t(const void* const* codes, int n, int k, uint16_t* ct, int64_t s_ct, int batch,
                          hipStream_t s);
hipError_t launch_mq(const MQArgs& a, int batch, hipStream_t s);
hipError_t launch_tall(const TallArgs& a, int batch, hipStream_t s);  // M_t^T P, B pre-split
hipError_t launch_split_t(const float* X, int64_t sX, int rows, int k, uint16_t* hi, uint16_t* lo, int64_t sT,
                          int batch, hipStream_t s);
hipError_t launch_split(const float* X, int64_t sX, int64_t count, uint16_t* hi, uint16_t* lo, int64_t sT, int batch,
                        hipStream_t s);
hipError_t launch_sum_pieces(const float* part, int pieces, int64_t count, float* out, int batch, hipStream_t s);
hipError_t launch_recon(const ReconArgs& a, int batch, hipStream_t s);
hipError_t launch_residual(const ResidualArgs& a, int batch, hipStream_t s);
hipError_t launch_gram(const CholArgs& a, int batch, hipStream_t s);
hipError_t launch_chol(const CholArgs& a, int batch, hipStream_t s);
hipError_t launch_row_solve(const CholArgs& a, int batch, hipStream_t s);
hipError_t launch_ptr_table(float* base, int64_t stride, int batch, float** out, hipStream_t s);

}  // namespace muon
