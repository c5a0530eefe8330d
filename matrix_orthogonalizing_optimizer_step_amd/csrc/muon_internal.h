// Internal declarations shared by the HIP kernels and the host schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Every workspace dimension is padded to a multiple of this, so the GEMM
// tiles never need bounds checks.  Padding rows/columns are kept at zero.
constexpr int kPad = 256;

// Operand (MFMA input) element types.
enum OpType : int { kOpF32 = 0, kOpBF16 = 1, kOpF16 = 2 };

// Storage dtypes of user buffers (values match muon_dtype).
enum DType : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Blocks per matrix for the norm / momentum reductions (fixed so the
// second stage sums a bounded, fixed-order list of partials).
constexpr int kNormBlocks = 512;

// Block tile edges of the MFMA kernels (16-bit operands) and of the fp32
// check path.
constexpr int kMfmaTile = 256;   // MFMA block tile: 256 rows by 256 (or kHalfTile) columns
constexpr int kHalfTile = 128;   // the narrow tile of short symmetric products
constexpr int kCheckTile = 64;

// One GEMM launch over a batch: C[i][j] = sum_k P[i][k] * Q[j][k] (both
// operands K-contiguous), followed by the fused epilogue
//   v = alpha * C + beta * E[i][j] + gamma * (i == j < n_real)
// with alpha/beta/gamma affine in the per-matrix diagonal shift a'.
struct GemmArgs {
  int Mdim, Ndim, K;   // padded problem size
  int n_real;          // real n: the diagonal term and the partial sums stop here
  int sym;             // 1: C symmetric, only lower tiles are computed and mirrored
  int ntiles;          // tiles per matrix in this launch
  int bn;              // MFMA kernels: block tile width, kMfmaTile or kHalfTile

  const void* P; int64_t sP; int ldp;  // row i of matrix b at P + b*sP + i*ldp
  const void* Q; int64_t sQ; int ldq;

  float alpha_c, alpha_a, beta_c, beta_a, gamma_c, gamma_a;
  float coef_a, coef_b, coef_c;        // a_t, b_t, c_t of this iteration
  const double* part_in; int npart_in; // (trace, sum of squares) per tile of the Gram matrix
  const float* shift_in;               // per-matrix a' from an earlier launch
  float* shift_out;                    // per-matrix a' written by tile 0

  const void* E16; int64_t sE; int lde;   // epilogue input E (operand type) or null

  void* out16; int64_t sO; int ldo;       // output (operand type and layout)
  void* outT16; int64_t sOT; int ldot;                     // transposed copy (non-symmetric only)
  void* q16;                              // v + a' I (a fresh Q), layout of out16
  double* part_out;                                        // (trace, sumsq) of v per tile

  int final_mode;                   // 1: v is O; update W and optionally store O
  void* const* W; int w_dtype;
  void* const* Oout; int o_dtype;
  int transposed;                   // user matrix is m x n (rows > cols)
  int m_real;                       // real m (columns of X)
  int user_ld;                      // leading dimension of the user's W / O
  float lr, wd, oscale;             // W <- W - lr (oscale O + wd W)

  // Tail split (MFMA kernels): the first full_blocks blocks each take a whole
  // tile; each of the remaining tiles (tiles beyond full_blocks, over the whole
  // batch) is cut along k into kpieces pieces, one block each.  The last piece
  // of a tile to finish adds the fp32 partials of all pieces in piece order
  // and runs the epilogue.  kpieces = 1: no split (full_blocks = all tiles).
  int full_blocks;
  int kpieces;
  float* part32;     // tail tiles x kpieces partial tiles (kMfmaTile^2 floats each)
  int* counters;     // one per tail tile, zero between launches
};

// Partial-tile storage of the tail split, per tile piece (floats).
constexpr int64_t kPartFloats = static_cast<int64_t>(kMfmaTile) * kMfmaTile;
// At most this many k pieces per tail tile.
constexpr int kMaxPieces = 8;

// Epilogue kinds of the MFMA kernel, one kernel instantiation each, so that
// every epilogue is straight-line code.
enum EpiKind : int {
  kEpiSym = 0,  // symmetric: C -> 16-bit (A or R = X X^T)
  kEpiSymE16,   // symmetric: v = alpha C + beta E + gamma I (B', Z', Q Z', R Z', Z' RZ)
  kEpiSymE16Q,  // as kEpiSymE16, plus a fresh Q = v + a' I
  kEpiGen,      // general: C -> X and X^T (Q X at a restart)
  kEpiGenE16,   // general: v = alpha C + beta X -> X and X^T (B X)
  kEpiFin,      // last product: O = C -> update of W
  kEpiFinE16,   // last product: O = alpha C + beta X -> update of W
  kNumEpiKinds
};

// The epilogue kind a launch's arguments ask for, or -1 if none matches.
int epi_kind(const GemmArgs& a);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_gemm(const GemmArgs& a, int batch, int op, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmArgs& a, int batch, int kind, hipStream_t s);
hipError_t launch_gemm_f16(const GemmArgs& a, int batch, int kind, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, int batch, hipStream_t s);
int gemm_tile(int op);  // block tile edge of the GEMM kernel used for an operand type

struct NormArgs {
  const void* const* M;   // user matrices
  int m_dtype;
  const void* const* G;   // gradients (momentum mode) or null
  void* const* Mw;        // momentum written back (momentum mode) or null
  double mu;
  int64_t count;          // rows * cols
  double* partials;       // batch * kNormBlocks
  int* zero;              // zero[0 .. nzero) is cleared by the kernel (GEMM tail counters)
  int nzero;
};
hipError_t launch_norm(const NormArgs& a, int batch, hipStream_t s);

struct PrepArgs {
  const void* const* M;  // user matrices (rows x cols)
  int m_dtype;
  int rows, cols;
  int transposed;        // X = M^T
  int n, m;              // real n, m
  int n_pad, m_pad;
  const double* partials;  // batch * kNormBlocks sums of squares
  double eps;
  void* XN; int64_t sXN;   // n_pad x m_pad, op type
  void* XT; int64_t sXT;   // m_pad x n_pad, op type
};
hipError_t launch_prep(const PrepArgs& a, int batch, int op, hipStream_t s);

}  // namespace muon
