/*
 * muon.h - C ABI of the MI355X (gfx950) Muon-step library.
 *
 * The Muon step for a 2-D weight matrix is: momentum M <- mu M + G, an
 * approximate polar factor O of M by Newton-Schulz iteration, and the weight
 * update W <- W - lr (O + wd W).  Sources, cited by short name:
 *
 *   [GNS]   "优化器 (3)（Gram Newton-Schulz）", blog notes on Gram Newton-Schulz
 *           (phycat-blog): §1.1 eq.(1) the step, §1.2 eq.(2) standard NS,
 *           §2.3 Alg.1 naive Gram NS, §3.2 restarts, §3.3 fp16 and eq.(13),
 *           §3.4 Alg.2 stabilised Gram NS.
 *   [GRASP] notes on "Achieving low-bit Muon through subspace preservation and
 *           grid quantization", overall framework: momentum, NS, update; the
 *           full example adds weight decay.
 *   [LiMuon] notes on LiMuon, design 3: the quintic (3.4445, -4.7750, 2.0315).
 *   [MuonBlog] "Muon Optimizer" blog post, §1: Muon is for 2-D matrices;
 *           §5 (Muon is no drop-in AdamW replacement) item 4: weight decay and
 *           a per-parameter update scale.
 *   [GRASP] also: key design 1 (top subspace P R^T kept in 8 bit, found by a
 *           warm-started power-iteration step), key design 2 (grid
 *           quantisation), the full example (the per-step flow) and the
 *           training strategy (INT4 / INT8, group and grid size 128).
 *
 * Conventions shared by every entry point:
 *
 *   Matrices are dense, row-major, contiguous (leading dimension = cols) and
 *   live in device memory.  A call works on a batch of `batch` matrices of one
 *   shape rows x cols; matrix arguments are DEVICE arrays of `batch` device
 *   pointers (one per matrix), so independent tensors can be batched.  The
 *   caller owns every buffer, including the workspace; the library allocates
 *   no device memory.  A matrix with rows > cols is iterated transposed
 *   ([GNS §1.2] works with n = min(rows, cols) <= m = max(rows, cols)); the
 *   result has the input's shape.
 *
 *   Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  Results are valid after the stream is synchronised.  Calls on
 *   one stream are ordered; calls that share a workspace must not overlap.
 *
 *   Errors: every argument is checked before anything is enqueued; on an
 *   error a status other than MUON_OK is returned and no buffer is touched.
 *   A failed launch returns MUON_ERR_HIP (buffers may then be partly written).
 *   Nothing is printed and nothing aborts.  NaN/Inf in the inputs propagate
 *   to the outputs.  A zero matrix gives O = 0 ([GNS §2.3 Alg.1]: eps keeps
 *   the normalisation finite).
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 6
#define MUON_MAX_T 16
#define MUON_MAX_DIM (1 << 20)
#define MUON_GRASP_MAX_K 1024

/* Element types.  F32 = IEEE binary32, BF16 = bfloat16, F16 = IEEE binary16. */
/* Each enum's last enumerator is no value to pass: it gives the type the range
 * of a 32-bit int, so the library can check any value a caller passes and
 * reject the ones it does not know (MUON_ERR_INVALID_ARG, "unknown status"). */
typedef enum { MUON_F32 = 0, MUON_BF16 = 1, MUON_F16 = 2, MUON_DTYPE_RANGE_ = 0x7fffffff } muon_dtype;

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1, /* bad shape, count, pointer, or parameter   */
  MUON_ERR_UNSUPPORTED = 2, /* a dtype combination the library lacks     */
  MUON_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required   */
  MUON_ERR_HIP = 4,         /* a HIP runtime call or launch failed       */
  MUON_STATUS_RANGE_ = 0x7fffffff
} muon_status;

typedef enum {
  MUON_NS_STANDARD = 0, /* [GNS §1.2 eq.(2)]                              */
  MUON_NS_GRAM = 1,     /* [GNS §2.3 Alg.1] / [GNS §3.4 Alg.2] (restarts) */
  MUON_NS_VARIANT_RANGE_ = 0x7fffffff
} muon_ns_variant;

/*
 * Newton-Schulz settings.  Fill with muon_ns_config_init() and change fields.
 *
 *   T            iterations, 1..MUON_MAX_T (the pages use 5).
 *   coeffs       HOST pointer to T*3 floats (a_t, b_t, c_t) for t = 1..T, read
 *                during the call only; NULL = (3.4445, -4.7750, 2.0315) for
 *                every t ([LiMuon design 3]).
 *   eps          X0 = X / (||X||_F + eps), default 1e-7 ([GNS §2.3 Alg.1]).
 *   restart_mask Gram only: bit (t-1) set = restart after iteration t ([GNS
 *                §3.2]); needs t < T.  Default 1u << 1 (after iteration 2, the
 *                choice of [GNS §3.2] and [GNS §3.4 Alg.2]); 0 = Alg.1.
 *                Ignored by the standard variant.
 *   compute      MFMA operand type: MUON_BF16 (standard default), MUON_F16
 *                (Gram default: [GNS §3.3] casts to float16), or MUON_F32 for
 *                the slow fp32 check path (fp32 operands, fp64 accumulation).
 *                Products always accumulate in fp32 or wider.  MUON_BF16 is
 *                accepted for the standard variant with the fixed quintic
 *                only; with the Gram variant or any other coefficient table
 *                every entry point returns MUON_ERR_UNSUPPORTED (and
 *                muon_workspace_size 0): bf16's 8-bit significand exceeds
 *                the 2e-2 relative error of the 16-bit path there, where
 *                MUON_F16, at the same MFMA rate, stays within it.
 *   shift        1 (default): each iteration splits its a_t I term into a
 *                diagonal shift a' (the mean of a_t + b_t l + c_t l^2 over the
 *                eigenvalues l of the Gram matrix, from its trace and
 *                Frobenius norm) that is applied in fp32, and the rest, which
 *                is folded into the 16-bit operand.  Exact in real arithmetic;
 *                it extends [GNS §3.3 eq.(13)] (keep the a_t arithmetic in
 *                fp32) and cuts 16-bit rounding error.  0 = plain a_t.
 */
typedef struct muon_ns_config {
  int32_t T;
  const float *coeffs;
  float eps;
  uint32_t restart_mask;
  muon_dtype compute;
  int32_t shift;
} muon_ns_config;

/* Defaults for a variant (see above).  `cfg` must not be NULL. */
void muon_ns_config_init(muon_ns_config *cfg, muon_ns_variant variant);

/*
 * Bytes of device workspace an orthogonalisation or step on `batch` matrices
 * of rows x cols needs (the same figure for ns_orthogonalize,
 * gram_ns_orthogonalize and muon_step with that variant).  Returns 0 when the
 * arguments are invalid.  cfg NULL = defaults.
 */
size_t muon_workspace_size(int batch, int rows, int cols, muon_ns_variant variant,
                           const muon_ns_config *cfg);

/*
 * Standard Newton-Schulz orthogonalisation [GNS §1.2 eq.(2)]:
 *   X0 = X / (||X||_F + eps); for t = 1..T: A = X X^T, B = b_t A + c_t A^2,
 *   X <- a_t X + B X; O = X_T.  Each matrix is normalised on its own.
 *
 *   M        device array of `batch` device pointers to rows x cols inputs of
 *            type m_dtype (F32, BF16 or F16).  Not modified.
 *   O        device array of `batch` device pointers to rows x cols outputs of
 *            type o_dtype (F32 or BF16); must not alias M.
 *   cfg      NULL = defaults of the standard variant.
 *   workspace, ws_bytes  device buffer of at least muon_workspace_size() bytes,
 *            256-byte aligned; contents on entry are ignored.
 */
muon_status ns_orthogonalize(int batch, int rows, int cols,
                             const void *const *M, muon_dtype m_dtype,
                             void *const *O, muon_dtype o_dtype,
                             const muon_ns_config *cfg,
                             void *workspace, size_t ws_bytes, void *stream);

/*
 * Gram Newton-Schulz orthogonalisation [GNS §2.3 Alg.1, §3.4 Alg.2]:
 *   R = X0 X0^T, Q = I; for t = 1..T: Z = b_t R + c_t R^2, Q <- Q Z + a_t Q,
 *   then a restart (X <- Q X, R = X X^T, Q = I) after the iterations in
 *   restart_mask, otherwise RZ = R Z + a_t R, R <- Z RZ + a_t RZ (not done at
 *   t = T); O = Q X.  Same arguments as ns_orthogonalize; cfg NULL = Gram
 *   defaults (fp16 operands, restart after iteration 2).
 */
muon_status gram_ns_orthogonalize(int batch, int rows, int cols,
                                  const void *const *M, muon_dtype m_dtype,
                                  void *const *O, muon_dtype o_dtype,
                                  const muon_ns_config *cfg,
                                  void *workspace, size_t ws_bytes, void *stream);

/*
 * One Muon step on a batch of same-shape weights ([GRASP framework], [GNS
 * §1.1 eq.(1)], [MuonBlog §1]):
 *   M <- mu M + G          (computed exactly in fp64, rounded to nearest even
 *                           into state_dtype; M is updated in place)
 *   O  = NS(M)             (variant and cfg as above, on the stored M)
 *   W <- W - lr (update_scale O + weight_decay W)
 *                          (fp32 arithmetic, W updated in place)
 *
 *   update_scale  the per-parameter update scale that [MuonBlog §5 item 4]
 *           names, with weight decay, as needed for large-scale training; the
 *           pages give no formula, so it is a plain factor chosen by the
 *           caller per call (per same-shape parameter group).  1 = the plain
 *           step of the other pages; it multiplies O in the update only
 *           (O_out receives O unscaled).  Must be finite.
 *
 *   W       device array of device pointers, rows x cols, w_dtype F32 or BF16.
 *   M       device array of device pointers, momentum, state_dtype F32 or
 *           BF16.  The first step of a run passes zeros (M_0 = 0).
 *   G       device array of device pointers, gradients, state_dtype.
 *   O_out   NULL, or a device array of device pointers that receive O in
 *           o_dtype (F32 or BF16), e.g. for checking.
 *   cfg     NULL = defaults of `variant`.
 * W, M, G and O_out must not alias one another.
 */
muon_status muon_step(int batch, int rows, int cols,
                      void *const *W, muon_dtype w_dtype,
                      void *const *M, const void *const *G, muon_dtype state_dtype,
                      float mu, float lr, float weight_decay, float update_scale,
                      muon_ns_variant variant, const muon_ns_config *cfg,
                      void *const *O_out, muon_dtype o_dtype,
                      void *workspace, size_t ws_bytes, void *stream);

/*
 * muon_step without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation).  It runs the same kernels as muon_step, with its
 * scratch memory in a fixed device array of MUON_FIXED_SCRATCH_BYTES inside
 * the library: one copy per device, allocated when the library's code is
 * loaded on that device and held until the process ends.  The call itself
 * allocates nothing; the caller still passes every input and output.
 *
 *   Arguments, checks and results as muon_step.  A problem whose workspace
 *   (muon_workspace_size for the same batch, shape, variant and cfg) exceeds
 *   MUON_FIXED_SCRATCH_BYTES is rejected with MUON_ERR_WORKSPACE before any
 *   device work.  The first call on a device looks up the array's address
 *   there (MUON_ERR_HIP if that fails).
 *   Every call on one device shares that device's array and leaves its
 *   contents behind: calls that overlap on one device (on different streams
 *   or from different threads without ordering) race and give wrong results.
 *   Order them on one stream, or use muon_step with separate workspaces.
 */
#define MUON_FIXED_SCRATCH_BYTES ((size_t)64 << 20)
muon_status muon_step_fixed_scratch(int batch, int rows, int cols,
                                    void *const *W, muon_dtype w_dtype,
                                    void *const *M, const void *const *G, muon_dtype state_dtype,
                                    float mu, float lr, float weight_decay, float update_scale,
                                    muon_ns_variant variant, const muon_ns_config *cfg,
                                    void *const *O_out, muon_dtype o_dtype, void *stream);

/*
 * Low-bit momentum state of 4-bit-Muon-GRASP ([GRASP] overall framework, key
 * designs 1 and 2, full example, training strategy).  The momentum of a
 * rows x cols weight is kept as M = M_res + P R^T with
 *
 *   M_res  4-bit grid code: the matrix is cut into 128 x 128 blocks (edge
 *          blocks cover the real rows and columns only); each block has a
 *          scale per row and per column, the largest magnitude of that row or
 *          column inside the block (NaN propagating).  An entry x is stored as
 *          q = rint(7 x / m), m = min(row scale, column scale), evaluated in
 *          fp64 from fp32 values, ties to even, q in -7..7 (q = 0 when m is 0,
 *          NaN or infinite), and restored as q m / 7.
 *   P, R   rows x k and cols x k factors of the top-k part in 8-bit group
 *          code: each row is cut into groups of 128 consecutive entries (the
 *          last one shorter) with scale = largest magnitude of the group; q =
 *          rint(127 x / scale) in fp64, restored as q scale / 127.
 *
 * Every field is a DEVICE array of `batch` device pointers, one per matrix:
 *   res_codes       uint8 [rows][(cols + 1) / 2]: two codes per byte along a
 *                   row, the even column in the low nibble (two's complement).
 *   res_row_scales  float [rows][ceil(cols / 128)]
 *   res_col_scales  float [ceil(rows / 128)][cols]
 *   P_codes         int8 [rows][k]     P_scales  float [rows][ceil(k / 128)]
 *   R_codes         int8 [cols][k]     R_scales  float [cols][ceil(k / 128)]
 * (the P and R fields are ignored when k = 0).  The caller owns the state.
 * Before the first step, the residual and P are zero (codes and scales) and R
 * holds the code of any cols x k start matrix, e.g. a Gaussian one (with P
 * zero, M_{-1} = 0 whatever R is, and R starts the power iteration).
 */
typedef struct muon_grasp_state {
  void *const *res_codes;
  void *const *res_row_scales;
  void *const *res_col_scales;
  void *const *P_codes;
  void *const *P_scales;
  void *const *R_codes;
  void *const *R_scales;
} muon_grasp_state;

/* Workspace bytes of muon_grasp_step (0 for invalid arguments). */
size_t muon_grasp_workspace_size(int batch, int rows, int cols, int k, muon_ns_variant variant,
                                 const muon_ns_config *cfg);

/*
 * One Muon step whose momentum lives in the low-bit state ([GRASP] full
 * example), for a batch of same-shape weights:
 *   M_{t-1} = deq(M_res) + deq(P) deq(R)^T
 *   M_t     = mu M_{t-1} + G      (fp64, rounded once to fp32)
 *   k > 0:  Q = R_{t-1} with unit columns (zero columns stay zero);
 *           P = QR Q factor of M_t Q (positive diagonal; a column dependent
 *           on the earlier ones, or zero, becomes zero); R = M_t^T P;
 *           P and R are stored in 8-bit code, M_res = M_t - P R^T in 4-bit
 *           grid code (P and R at full precision in the residual).
 *   k = 0:  no subspace: M_t itself is stored in 4-bit grid code.
 *   O = NS(M_t) (variant, cfg as for muon_step), W <- W - lr (update_scale O
 *   + weight_decay W).
 *
 *   k        subspace rank, 0 <= k <= min(rows, cols), k <= MUON_GRASP_MAX_K
 *            ([GRASP] uses rank / 16).  batch <= 8191.
 *   state    see muon_grasp_state; updated in place.
 *   G        gradients (F32, BF16 or F16).  W: F32 or BF16, updated in place.
 *   O_out    NULL or outputs for O (F32 or BF16).
 *   M_out    NULL or F32 outputs that receive M_t (for checking).
 * W, G, O_out and M_out must be distinct arrays (MUON_ERR_INVALID_ARG).
 *   aux_stream  NULL, or a second stream of the caller's on the same device:
 *            with k > 0 the update of the state (everything after M_t: the
 *            power iteration, the codes of P and R, the residual) then runs
 *            there, beside Newton-Schulz on `stream`, from an event recorded
 *            on `stream`; the call ends by making `stream` wait for it, so the
 *            whole step is complete when `stream` passes the call.  Other work
 *            on aux_stream must not touch the state or the workspace meanwhile.
 * The products with fp32 operands (M_t Q, M_t^T P, P R^T) run on the bf16
 * MFMA with each operand split into two bf16 parts (about 16 significant bits
 * per product); the Gram matrix P~^T P~, its Cholesky factor and the solve
 * P = P~ U^{-1} are fp64.  Errors as for muon_step.
 */
muon_status muon_grasp_step(int batch, int rows, int cols, int k,
                            void *const *W, muon_dtype w_dtype,
                            const muon_grasp_state *state,
                            const void *const *G, muon_dtype g_dtype,
                            float mu, float lr, float weight_decay, float update_scale,
                            muon_ns_variant variant, const muon_ns_config *cfg,
                            void *const *O_out, muon_dtype o_dtype, void *const *M_out,
                            void *workspace, size_t ws_bytes, void *stream, void *aux_stream);

/*
 * The two codes on their own ([GRASP] key design 2, training strategy), with
 * the layouts above; device arrays of device pointers, fp32 values.  Grid
 * code: X and Y are rows x cols; group code: X and Y are rows x k.  batch <= 65535.
 */
muon_status muon_grid_quantize(int batch, int rows, int cols, const void *const *X, void *const *codes,
                               void *const *row_scales, void *const *col_scales, void *stream);
muon_status muon_grid_dequantize(int batch, int rows, int cols, const void *const *codes,
                                 const void *const *row_scales, const void *const *col_scales,
                                 void *const *Y, void *stream);
muon_status muon_group8_quantize(int batch, int rows, int k, const void *const *X, void *const *codes,
                                 void *const *scales, void *stream);
muon_status muon_group8_dequantize(int batch, int rows, int k, const void *const *codes,
                                   const void *const *scales, void *const *Y, void *stream);

/*
 * Per-iteration coefficient schedule in the manner of the Polar Express
 * quintics that [GNS §3.2] iterates with (its printed table is garbled, so
 * the schedule is derived from the method's principle rather than copied):
 * p_t(x) = a_t x + b_t x^3 + c_t x^5 is the odd quintic nearest to 1 in the
 * maximum norm on [l_t, u_t], the interval that holds the singular values of
 * X_{t-1} when those of X0 lie in [ell, 1]; [l_{t+1}, u_{t+1}] is the image of
 * [l_t, u_t] under the applied polynomial.  The [GNS §3.3] safety factor f
 * applies each polynomial as p_t(x / f), i.e. (a_t / f, b_t / f^3, c_t / f^5),
 * so singular values somewhat above the design range still converge.  Once
 * (u_t - l_t) / u_t <= 1e-2 the minimax polynomials are replaced by their
 * limit (15/8, -10/8, 3/8) (p(1) = 1, p'(1) = p''(1) = 0; its error there is
 * below 3e-6, under any 16-bit rounding).  The coefficients
 * are rounded to fp32, and the intervals follow the rounded polynomials.
 *
 * Use with Gram NS: the schedule (T = 5, ell = 1e-3, f = 1 or 1.05) was
 * checked with the Gram default, one restart after iteration 2.  By the
 * diagnostics [GNS §3.2] judges restarts with (the smallest eigenvalue of
 * every Gram matrix, the condition number of Q_t), with Gram matrices
 * rounded to bf16 or holding a spurious eigenvalue of -1e-5 ([GNS §3.1]),
 * that is the single restart point that keeps the eigenvalues above -0.4
 * and gives the best-conditioned Q on square Gaussian inputs (cond below
 * 100 there and on rectangular ones); without a restart the spurious
 * eigenvalue grows past -1.  The steep first polynomial (a_1 ~ 8) can leave
 * cond(Q_2) near 170 on inputs whose singular values fill [ell, 1] (e.g.
 * sigma_i ~ i^-1/2), whatever the restart point.  bf16 operands refuse
 * such a table (see muon_ns_config.compute); use MUON_F16.
 *
 *   T       iterations, 1..MUON_MAX_T.
 *   ell     lower end of the singular values of X0, 0 < ell < 1 (e.g. 1e-3).
 *   safety  f, 1 <= f <= 2 (1 = none; [GNS §3.3] uses 1.05).
 *   coeffs  HOST array of 3 T floats receiving (a_t, b_t, c_t), t = 1..T, in
 *           the layout muon_ns_config.coeffs reads.
 *   bounds  NULL, or a HOST array of 2 T + 2 doubles receiving l_1, u_1 (=
 *           ell, 1), l_2, u_2, ..., l_{T+1}, u_{T+1}.
 * Host-only arithmetic (no device, no stream).  Returns MUON_ERR_INVALID_ARG
 * for arguments out of range, MUON_ERR_UNSUPPORTED if the minimax exchange
 * does not settle (not observed for 1e-7 <= ell < 1); outputs are then
 * partly written.
 */
muon_status muon_quintic_schedule(int T, double ell, double safety, float *coeffs, double *bounds);

/*
 * Floating-point operations of one orthogonalisation of a rows x cols matrix
 * ([GNS §1.2], §2.4, §3.4).  symmetric_aware = 1 counts half for products
 * whose result is symmetric (only one triangle is computed): standard NS
 * T(3 alpha + 1) n^3, Gram NS (17 + 3 alpha) n^3 with no restart and
 * (14 + 6 alpha) n^3 with one restart at T = 5.  symmetric_aware = 0 gives the
 * dense-equivalent count ((20 alpha + 10) n^3 for standard NS at T = 5).
 * Returns 0 for invalid arguments.
 */
double muon_ns_flops(int rows, int cols, muon_ns_variant variant,
                     const muon_ns_config *cfg, int symmetric_aware);

/*
 * Opt-in launch trace, for profiling.  While enabled, every kernel the
 * library launches is bracketed by two hipEvents recorded on the call's
 * stream, and tagged with its kernel, its role in the iteration and its
 * algorithmic work: FLOPs (symmetric products count one triangle) and bytes
 * (each operand read once, each output written once).  The library keeps this
 * one piece of process-wide state; enabling or disabling clears it.
 */
typedef struct muon_trace_record {
  char kernel[40]; /* kernel symbol family, e.g. "gemm_nt_mfma_f16"      */
  char role[24];   /* e.g. "XXt", "A2", "BX", "ZRZ", "momentum_norm"     */
  double flops;    /* algorithmic floating-point operations              */
  double bytes;    /* algorithmic HBM bytes                              */
  float ms;        /* measured duration between the two events           */
} muon_trace_record;

/* Turn the trace on (1) or off (0); returns the previous setting. */
int muon_trace_enable(int enable);

/*
 * Wait for the recorded events, copy up to `max` records (oldest first) into
 * `out` (may be NULL with max = 0) and return how many were recorded.  The
 * records are then cleared.  Returns -1 if a HIP event call failed.
 */
int muon_trace_collect(muon_trace_record *out, int max);

/*
 * Practical 16-bit MFMA ceiling of the device, for profiling beside the
 * launch trace.  Launches `blocks` blocks of 256 threads on `stream`; every
 * wave issues 32 * rounds v_mfma_f32_32x32x16 instructions of operand type
 * `dtype` (MUON_F16 or MUON_BF16; 32768 FLOPs each) on register operands
 * only, whose values come from a fixed hash so that they switch like real
 * data, and each thread finally stores one float to sink[block * 256 +
 * thread] (`sink`: device buffer of blocks * 256 floats, owned by the
 * caller; its contents are meaningless).  The caller times the launch with
 * events on the same stream: FLOPs = blocks * 4 * 32 * rounds * 32768.
 * Under a full MFMA load the clock is set by the power the data draw, so
 * this rate, not the dense peak at the nominal clock, bounds what any GEMM of
 * that operand type reaches.  Returns MUON_ERR_INVALID_ARG for blocks outside
 * [1, 2^20], rounds < 1, another dtype or a NULL sink (nothing launched),
 * MUON_ERR_HIP if the launch fails.
 */
muon_status muon_mfma_ceiling(int blocks, int rounds, muon_dtype dtype, float *sink, void *stream);

/* Static description of a status code (never NULL). */
const char *muon_status_string(muon_status status);

/* MUON_ABI_VERSION of the loaded library. */
int muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
