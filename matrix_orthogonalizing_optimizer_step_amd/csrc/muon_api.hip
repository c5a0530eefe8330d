// Host side of the C ABI in include/muon.h: argument checks, workspace
// layout and the launch schedule of the standard and Gram Newton-Schulz
// iterations.  All work is enqueued on the caller's stream; nothing blocks.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/muon.h"
#include "muon_grasp.h"
#include "muon_internal.h"

using namespace muon;

namespace {

constexpr float kQuintic[3] = {3.4445f, -4.7750f, 2.0315f};  // [LiMuon design 3]

struct Config {
  int T;
  float c[MUON_MAX_T][3];
  double eps;
  uint32_t restart_mask;
  int op;
  int shift;
};

struct Plan {
  int batch, rows, cols;
  int n, m, n_pad, m_pad, transposed;
  int op, esz, tile;
  muon_ns_variant variant;
  size_t XN, XT[2];
  size_t A16, B16;                                        // standard
  size_t R16, Z16, RZ16, Q16[2];                         // Gram
  size_t normpart, tilepart, shift;
  size_t part32, counters;                               // tail split of the MFMA GEMMs
  int cu;                                                // compute units the split is planned for
  int max_tail, max_pieces;                              // largest tail over the launches of a call
  size_t total;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Tail split of a GEMM launch of `tiles` tiles with k in `units` units of
// 256 on `cu` compute units: whole tiles fill the complete rounds, and the
// tiles of the last, partial round are cut into as many k pieces as the idle
// compute units allow (at most kMaxPieces).  Only long products are split
// (k of at least 8192, pieces of at least 1024): handing a partial tile over
// costs a device-scope fence (an L2 write-back) and an fp32 round trip, which
// shorter tiles do not amortise (measured: a net loss at k = 3584).
#ifndef MUON_TAIL_MIN_UNITS
#define MUON_TAIL_MIN_UNITS 32
#endif
constexpr int kTailMinUnits = MUON_TAIL_MIN_UNITS;

void tail_split(int64_t tiles, int units, int cu, int* full, int* pieces) {
  const int64_t rounds = tiles / cu, tail = tiles - rounds * cu;
  int s = tail > 0 && units >= kTailMinUnits ? static_cast<int>(cu / tail) : 1;
  s = s < kMaxPieces ? s : kMaxPieces;
  s = s < units / 4 ? s : units / 4;
  if (s < 2) {
    *full = static_cast<int>(tiles);
    *pieces = 1;
  } else {
    *full = static_cast<int>(rounds * cu);
    *pieces = s;
  }
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) return 256;
  return n;
}

// ---------------------------------------------------------------------------
// opt-in launch trace (muon_trace_enable / muon_trace_collect)
// ---------------------------------------------------------------------------
struct TraceRec {
  muon_trace_record rec;
  hipEvent_t e0, e1;
};

struct Trace {
  std::mutex mu;
  bool on = false;
  std::vector<TraceRec> recs;
  std::vector<hipEvent_t> pool;
} g_trace;

hipEvent_t trace_event() {  // caller holds g_trace.mu
  if (!g_trace.pool.empty()) {
    hipEvent_t e = g_trace.pool.back();
    g_trace.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void copy_name(char* dst, size_t n, const char* src) {
  strncpy(dst, src, n - 1);
  dst[n - 1] = '\0';
}

template <class F>
hipError_t traced(hipStream_t s, const char* kernel, const char* role, double flops, double bytes,
                  F&& launch) {
  if (!g_trace.on) return launch();
  std::lock_guard<std::mutex> lock(g_trace.mu);
  TraceRec r;
  memset(&r.rec, 0, sizeof(r.rec));
  copy_name(r.rec.kernel, sizeof(r.rec.kernel), kernel);
  copy_name(r.rec.role, sizeof(r.rec.role), role);
  r.rec.flops = flops;
  r.rec.bytes = bytes;
  r.e0 = trace_event();
  r.e1 = trace_event();
  if (r.e0 == nullptr || r.e1 == nullptr) return hipErrorOutOfMemory;
  hipError_t err = hipEventRecord(r.e0, s);
  if (err != hipSuccess) return err;
  err = launch();
  if (err != hipSuccess) return err;
  err = hipEventRecord(r.e1, s);
  if (err != hipSuccess) return err;
  g_trace.recs.push_back(r);
  return hipSuccess;
}

// The kernel a GEMM launch runs, spelled as the profiler prints it, so the
// launch trace and a rocprofv3 summary name the same kernels.
void gemm_kernel_name(const GemmArgs& g, int op, char* out, size_t n) {
  if (op == kOpF32) {
    snprintf(out, n, "gemm_nt_f64acc");
  } else {
    snprintf(out, n, "gemm_nt_mfma<%d, %d, %d>", op, epi_kind(g), g.bn);
  }
}

bool valid_dtype(muon_dtype d) { return d == MUON_F32 || d == MUON_BF16 || d == MUON_F16; }

muon_status make_config(const muon_ns_config* user, muon_ns_variant v, Config* out) {
  muon_ns_config cfg;
  if (user != nullptr) {
    cfg = *user;
  } else {
    muon_ns_config_init(&cfg, v);
  }
  if (cfg.T < 1 || cfg.T > MUON_MAX_T) return MUON_ERR_INVALID_ARG;
  if (!(cfg.eps >= 0.0f) || !isfinite(cfg.eps)) return MUON_ERR_INVALID_ARG;
  if (cfg.shift != 0 && cfg.shift != 1) return MUON_ERR_INVALID_ARG;
  if (!valid_dtype(cfg.compute)) return MUON_ERR_INVALID_ARG;
  if (v == MUON_NS_GRAM && (cfg.restart_mask >> (cfg.T - 1)) != 0u) return MUON_ERR_INVALID_ARG;
  out->T = cfg.T;
  bool quintic = true;  // the fixed quintic for every t
  for (int t = 0; t < cfg.T; ++t) {
    for (int k = 0; k < 3; ++k) {
      const float x = cfg.coeffs != nullptr ? cfg.coeffs[3 * t + k] : kQuintic[k];
      if (!isfinite(x)) return MUON_ERR_INVALID_ARG;
      out->c[t][k] = x;
      quintic = quintic && x == kQuintic[k];
    }
  }
  // bf16 operands (8 significant bits) stay within the 2e-2 relative error
  // of the 16-bit path only for standard NS with the fixed quintic.  Gram NS
  // computes in float16 ([GNS §3.3], [GNS §3.4 Alg.2]): with bf16 operands
  // square matrices (singular values down to ~n^-1.5 of the norm) measure
  // 2-3.5e-2.  Steep per-iteration polynomials (a_1 ~ 8.5 in the derived
  // minimax schedules) amplify bf16 rounding past the tolerance as well
  // (up to 2.6e-2 standard, 1.05e-1 Gram); float16 operands, at the same
  // MFMA rate, hold both.
  if (cfg.compute == MUON_BF16 && (v == MUON_NS_GRAM || !quintic)) return MUON_ERR_UNSUPPORTED;
  out->eps = cfg.eps;
  out->restart_mask = v == MUON_NS_GRAM ? cfg.restart_mask : 0u;
  out->op = cfg.compute == MUON_F32 ? kOpF32 : (cfg.compute == MUON_BF16 ? kOpBF16 : kOpF16);
  out->shift = cfg.shift;
  return MUON_OK;
}

// Workspace layout; returns false on invalid shapes or size overflow.
bool make_plan(int batch, int rows, int cols, muon_ns_variant v, const Config& c, Plan* p) {
  if (batch < 1 || rows < 1 || cols < 1 || rows > MUON_MAX_DIM || cols > MUON_MAX_DIM) return false;
  if (v != MUON_NS_STANDARD && v != MUON_NS_GRAM) return false;
  memset(p, 0, sizeof(*p));
  p->batch = batch;
  p->rows = rows;
  p->cols = cols;
  p->transposed = rows > cols;
  p->n = p->transposed ? cols : rows;
  p->m = p->transposed ? rows : cols;
  p->n_pad = static_cast<int>(round_up(p->n, kPad));
  p->m_pad = static_cast<int>(round_up(p->m, kPad));
  p->op = c.op;
  p->esz = c.op == kOpF32 ? 4 : 2;
  p->tile = gemm_tile(c.op);
  p->variant = v;
  const double bytes_x = static_cast<double>(batch) * p->n_pad * p->m_pad * p->esz;
  const double bytes_nn = static_cast<double>(batch) * p->n_pad * p->n_pad;
  if (bytes_x * 3 + bytes_nn * 24 > 4.0e14) return false;  // far beyond any device
  // the GEMM addresses one operand matrix with 32-bit byte offsets
  if (static_cast<double>(p->n_pad) * p->m_pad * p->esz >= 2147483648.0) return false;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = round_up(cur + bytes, 256);
    return at;
  };
  const size_t nx = static_cast<size_t>(batch) * p->n_pad * p->m_pad;
  const size_t nn = static_cast<size_t>(batch) * p->n_pad * p->n_pad;
  p->XN = take(nx * p->esz);
  p->XT[0] = take(nx * p->esz);
  p->XT[1] = take(nx * p->esz);
  if (v == MUON_NS_STANDARD) {
    p->A16 = take(nn * p->esz);
    p->B16 = take(nn * p->esz);
  } else {
    p->R16 = take(nn * p->esz);
    p->Z16 = take(nn * p->esz);
    p->RZ16 = take(nn * p->esz);
    p->Q16[0] = take(nn * p->esz);
    p->Q16[1] = take(nn * p->esz);
  }
  const int nt = p->n_pad / p->tile;
  p->normpart = take(static_cast<size_t>(batch) * kNormBlocks * sizeof(double));
  // (trace, sum of squares) per tile of a symmetric product, in 256 x 128 tiles at most
  p->tilepart = take(static_cast<size_t>(batch) * nt * (nt + 1) * 2 * sizeof(double));
  p->shift = take(static_cast<size_t>(batch) * sizeof(float));
  // the tail split's partial tiles and counters, sized for the largest tail
  // of this call's launches (symmetric K = m or n, general K = n)
  p->cu = p->op == kOpF32 ? 0 : device_cus();
  p->max_tail = 0;
  p->max_pieces = 0;
  if (p->cu > 0) {
    const int64_t tri = static_cast<int64_t>(batch) * nt * (nt + 1) / 2;
    const int64_t gen = static_cast<int64_t>(batch) * nt * (p->m_pad / p->tile);
    const struct { int64_t tiles; int units; } launches[3] = {
        {tri, p->m_pad / 256}, {tri, p->n_pad / 256}, {gen, p->n_pad / 256}};
    for (const auto& l : launches) {
      int full = 0, pieces = 1;
      tail_split(l.tiles, l.units, p->cu, &full, &pieces);
      if (pieces > 1) {
        const int tail = static_cast<int>(l.tiles - full);
        p->max_tail = tail > p->max_tail ? tail : p->max_tail;
        p->max_pieces = tail * pieces > p->max_pieces ? tail * pieces : p->max_pieces;
      }
    }
  }
  p->part32 = take(static_cast<size_t>(p->max_pieces) * kPartFloats * sizeof(float));
  p->counters = take(static_cast<size_t>(p->max_tail) * sizeof(int));
  p->total = cur;
  return true;
}

GemmArgs base_args(const Plan& p, char* ws) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.n_real = p.n;
  g.m_real = p.m;
  g.alpha_c = 1.0f;
  g.kpieces = 1;
  g.part32 = reinterpret_cast<float*>(ws + p.part32);
  g.counters = reinterpret_cast<int*>(ws + p.counters);
  return g;
}

// Symmetric MFMA products with k up to this may use 256 x 128 tiles (two
// blocks per compute unit); longer ones keep 256 x 256 tiles, whose deeper P
// look-ahead covers operands streamed from HBM.
constexpr int kHalfTileMaxK = 4096;

// Whether T whole tiles on `cu` compute units finish sooner as 2 T half
// tiles.  In units of one whole tile's time on a compute unit: whole tiles
// take ceil(T / cu) rounds; half tiles run two per compute unit (a pair takes
// about one unit) and a last round of at most one half tile per compute unit
// takes about 0.6 (one wave per SIMD again).  So the half tiles gain when the
// last round of whole tiles is at most half full, and tie otherwise (measured:
// three 3584^2 products, 315 tiles, +25 %; two, 210 tiles, -1 %).
bool half_tiles_pay(int64_t T, int cu) {
  const int64_t r = T % cu;
  return r > 0 && 2 * r <= cu;
}

// C = P P^T-style symmetric product of two n_pad x n_pad (or n_pad x K) operands.
void set_sym(GemmArgs& g, const Plan& p, const void* P, const void* Q, int K, int64_t sPQ, int ld) {
  g.Mdim = g.Ndim = p.n_pad;
  g.K = K;
  g.sym = 1;
  g.P = P;
  g.Q = Q;
  g.sP = g.sQ = sPQ;
  g.ldp = g.ldq = ld;
  const int nt = p.n_pad / p.tile;
  g.bn = kMfmaTile;
  g.ntiles = nt * (nt + 1) / 2;
  if (p.op != kOpF32 && K <= kHalfTileMaxK && half_tiles_pay(static_cast<int64_t>(g.ntiles) * p.batch, p.cu)) {
    // the lower triangle in 256 x 128 tiles: 2 I + 2 of them in tile row I
    g.bn = kHalfTile;
    g.ntiles = nt * (nt + 1);
  }
  g.sO = static_cast<int64_t>(p.n_pad) * p.n_pad;
  g.ldo = p.n_pad;
  g.sE = g.sO;
  g.lde = p.n_pad;
}

// C = P X with P an n_pad x n_pad operand and X given as X^T (m_pad x n_pad).
void set_px(GemmArgs& g, const Plan& p, const void* P, const void* XT) {
  g.Mdim = p.n_pad;
  g.Ndim = p.m_pad;
  g.K = p.n_pad;
  g.sym = 0;
  g.P = P;
  g.sP = static_cast<int64_t>(p.n_pad) * p.n_pad;
  g.ldp = p.n_pad;
  g.Q = XT;
  g.sQ = static_cast<int64_t>(p.m_pad) * p.n_pad;
  g.ldq = p.n_pad;
  g.bn = kMfmaTile;
  g.ntiles = (p.n_pad / p.tile) * (p.m_pad / p.tile);
  g.sO = static_cast<int64_t>(p.n_pad) * p.m_pad;
  g.ldo = p.m_pad;
  g.sE = g.sO;
  g.lde = p.m_pad;
  g.sOT = static_cast<int64_t>(p.m_pad) * p.n_pad;
  g.ldot = p.n_pad;
}

struct Final {
  void* const* W;
  int w_dtype;
  void* const* O;
  int o_dtype;
  float lr, wd, oscale;
};

void set_final(GemmArgs& g, const Plan& p, const Final& f) {
  g.final_mode = 1;
  g.W = f.W;
  g.w_dtype = f.w_dtype;
  g.Oout = f.O;
  g.o_dtype = f.o_dtype;
  g.transposed = p.transposed;
  g.user_ld = p.cols;
  g.lr = f.lr;
  g.wd = f.wd;
  g.oscale = f.oscale;
  if (p.op != kOpF32 && g.K <= kHalfTileMaxK) {
    // 256 x 128 tiles, two blocks per compute unit: the update of W (HBM-bound)
    // in one block's epilogue overlaps the other block's MFMAs.  Measured: the
    // last product of three 3584x18944 matrices 1.84 -> 1.67 ms; the other
    // products of X, whose epilogue writes only 16-bit X and X^T, are slower
    // in narrow tiles
    g.bn = kHalfTile;
    g.ntiles = (p.n_pad / p.tile) * (p.m_pad / kHalfTile);
  }
}

#define MUON_LAUNCH(expr)                        \
  do {                                           \
    if ((expr) != hipSuccess) return MUON_ERR_HIP; \
  } while (0)

// One GEMM launch with its algorithmic work for the trace: a symmetric
// product counts one triangle (n^2 K FLOPs), a general one 2 n m K; bytes are
// each operand read once plus each output written once (real sizes).
hipError_t gemm(const Plan& p, GemmArgs g, const char* role, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>(g.ntiles) * p.batch;
  g.full_blocks = static_cast<int>(tiles);
  g.kpieces = 1;
  if (p.cu > 0 && g.bn == kMfmaTile) {
    int full = 0, pieces = 1;
    tail_split(tiles, g.K / 256, p.cu, &full, &pieces);
    if (pieces > 1 && (tiles - full) <= p.max_tail && (tiles - full) * pieces <= p.max_pieces) {
      g.full_blocks = full;
      g.kpieces = pieces;
    }
  }
  const double n = p.n, m = p.m, esz = p.esz;
  double flops, bytes;
  if (g.sym) {
    const double K = g.K == p.m_pad ? m : n;
    flops = n * n * K;
    bytes = (g.P == g.Q ? 1.0 : 2.0) * n * K * esz;
    if (g.E16 != nullptr && g.E16 != g.P && g.E16 != g.Q) bytes += n * n * esz;
    if (g.out16 != nullptr) bytes += n * n * esz;
    if (g.q16 != nullptr) bytes += n * n * esz;
  } else {
    flops = 2.0 * n * n * m;
    bytes = n * n * esz + n * m * esz;
    if (g.E16 != nullptr) bytes += n * m * esz;
    if (g.out16 != nullptr) bytes += n * m * esz;
    if (g.outT16 != nullptr) bytes += n * m * esz;
    if (g.final_mode) {
      const double wsz = g.w_dtype == kF32 ? 4 : 2;
      if (g.W != nullptr) bytes += 2 * n * m * wsz;
      if (g.Oout != nullptr) bytes += n * m * (g.o_dtype == kF32 ? 4 : 2);
    }
  }
  if (g.final_mode) role = strcmp(role, "BX") == 0 ? "BX_final" : "QX_final";
  char kname[40];
  gemm_kernel_name(g, p.op, kname, sizeof(kname));
  return traced(s, kname, role, flops * p.batch, bytes * p.batch,
                [&] { return launch_gemm(g, p.batch, p.op, s); });
}

// Norm (and momentum), then X0 in both layouts.
muon_status run_prologue(const Plan& p, const Config& c, char* ws, const void* const* M, int m_dtype,
                         const void* const* G, void* const* Mw, double mu, hipStream_t s) {
  NormArgs na;
  na.M = M;
  na.m_dtype = m_dtype;
  na.G = G;
  na.Mw = Mw;
  na.mu = mu;
  na.count = static_cast<int64_t>(p.rows) * p.cols;
  na.partials = reinterpret_cast<double*>(ws + p.normpart);
  na.zero = reinterpret_cast<int*>(ws + p.counters);
  na.nzero = p.max_tail;
  {
    const double cnt = static_cast<double>(na.count) * p.batch;
    const double esz_m = m_dtype == kF32 ? 4 : 2;
    const double bytes = cnt * esz_m * (G != nullptr ? 3.0 : 1.0);
    char kname[40];
    snprintf(kname, sizeof(kname), "norm_kernel<%d>", m_dtype);
    MUON_LAUNCH(traced(s, kname, G != nullptr ? "momentum_norm" : "norm", 0.0, bytes,
                       [&] { return launch_norm(na, p.batch, s); }));
  }
  PrepArgs pa;
  pa.M = Mw != nullptr ? reinterpret_cast<const void* const*>(Mw) : M;
  pa.m_dtype = m_dtype;
  pa.rows = p.rows;
  pa.cols = p.cols;
  pa.transposed = p.transposed;
  pa.n = p.n;
  pa.m = p.m;
  pa.n_pad = p.n_pad;
  pa.m_pad = p.m_pad;
  pa.partials = na.partials;
  pa.eps = c.eps;
  pa.XN = ws + p.XN;
  pa.sXN = static_cast<int64_t>(p.n_pad) * p.m_pad;
  pa.XT = ws + p.XT[0];
  pa.sXT = pa.sXN;
  {
    const double cnt = static_cast<double>(p.n) * p.m * p.batch;
    const double bytes = cnt * ((m_dtype == kF32 ? 4 : 2) + 2.0 * p.esz);
    char kname[40];
    if (p.op == kOpF32) {
      snprintf(kname, sizeof(kname), "prep_f32_kernel<%d>", m_dtype);
    } else {
      snprintf(kname, sizeof(kname), "prep_packed_kernel<%d, %d>", m_dtype, p.op);
    }
    MUON_LAUNCH(traced(s, kname, "prep", 0.0, bytes, [&] { return launch_prep(pa, p.batch, p.op, s); }));
  }
  return MUON_OK;
}

// Standard Newton-Schulz ([GNS §1.2 eq.(2)]): per iteration A = X X^T,
// B' = c A^2 + b A + (a - a') I, X <- a' X + B' X (a' = a without the shift).
muon_status run_standard(const Plan& p, const Config& c, char* ws, const Final& f, hipStream_t s) {
  const int64_t sx = static_cast<int64_t>(p.n_pad) * p.m_pad;
  const int64_t snn = static_cast<int64_t>(p.n_pad) * p.n_pad;
  double* tp = reinterpret_cast<double*>(ws + p.tilepart);
  float* shift = reinterpret_cast<float*>(ws + p.shift);
  int xc = 0;
  for (int t = 0; t < c.T; ++t) {
    const float a = c.c[t][0], b = c.c[t][1], cc = c.c[t][2];
    // A = X X^T
    GemmArgs g = base_args(p, ws);
    set_sym(g, p, ws + p.XN, ws + p.XN, p.m_pad, sx, p.m_pad);
    g.out16 = ws + p.A16;
    g.part_out = c.shift ? tp : nullptr;
    const int npart = g.ntiles;  // partials of A, one per tile of this launch
    MUON_LAUNCH(gemm(p, g, "XXt", s));
    // B' = c A A + b A + (a - a') I
    g = base_args(p, ws);
    set_sym(g, p, ws + p.A16, ws + p.A16, p.n_pad, snn, p.n_pad);
    g.alpha_c = cc;
    g.E16 = ws + p.A16;
    g.beta_c = b;
    g.gamma_c = a;
    g.gamma_a = -1.0f;
    g.coef_a = a;
    g.coef_b = b;
    g.coef_c = cc;
    if (c.shift) {
      g.part_in = tp;
      g.npart_in = npart;
      g.shift_out = shift;
    }
    g.out16 = ws + p.B16;
    MUON_LAUNCH(gemm(p, g, "A2", s));
    // X <- a' X + B' X
    g = base_args(p, ws);
    set_px(g, p, ws + p.B16, ws + p.XT[xc]);
    if (p.op == kOpF32) {
      g.E16 = ws + p.XN;
    } else {  // the MFMA epilogue reads the a' X term from X^T
      g.E16 = ws + p.XT[xc];
      g.lde = p.n_pad;
    }
    g.beta_a = 1.0f;
    g.coef_a = a;
    g.shift_in = c.shift ? shift : nullptr;
    if (t + 1 < c.T) {
      g.out16 = ws + p.XN;
      g.outT16 = ws + p.XT[xc ^ 1];
      xc ^= 1;
    } else {
      set_final(g, p, f);
    }
    MUON_LAUNCH(gemm(p, g, "BX", s));
  }
  return MUON_OK;
}

// Gram Newton-Schulz ([GNS §2.3 Alg.1], [GNS §3.4 Alg.2]) with restarts.
muon_status run_gram(const Plan& p, const Config& c, char* ws, const Final& f, hipStream_t s) {
  const int64_t sx = static_cast<int64_t>(p.n_pad) * p.m_pad;
  double* tp = reinterpret_cast<double*>(ws + p.tilepart);
  float* shift = reinterpret_cast<float*>(ws + p.shift);
  char* R16 = ws + p.R16;
  char* Z16 = ws + p.Z16;
  char* RZ16 = ws + p.RZ16;
  const int64_t snn = static_cast<int64_t>(p.n_pad) * p.n_pad;
  int xc = 0, qc = 0;
  int npart = 0;  // tiles (one partial each) of the launch that last wrote R

  auto gram_of_x = [&]() {  // R = X X^T + partials
    GemmArgs g = base_args(p, ws);
    set_sym(g, p, ws + p.XN, ws + p.XN, p.m_pad, sx, p.m_pad);
    g.out16 = R16;
    g.part_out = c.shift ? tp : nullptr;
    npart = g.ntiles;
    return gemm(p, g, "XXt", s);
  };
  MUON_LAUNCH(gram_of_x());
  bool fresh = true;
  for (int t = 1; t <= c.T; ++t) {
    const float a = c.c[t - 1][0], b = c.c[t - 1][1], cc = c.c[t - 1][2];
    // Z' = c R R + b R + (a - a') I; a fresh Q becomes Z' + a' I
    GemmArgs g = base_args(p, ws);
    set_sym(g, p, R16, R16, p.n_pad, snn, p.n_pad);
    g.alpha_c = cc;
    g.E16 = R16;
    g.beta_c = b;
    g.gamma_c = a;
    g.gamma_a = -1.0f;
    g.coef_a = a;
    g.coef_b = b;
    g.coef_c = cc;
    if (c.shift) {
      g.part_in = tp;
      g.npart_in = npart;
      g.shift_out = shift;
    }
    g.out16 = Z16;
    if (fresh) g.q16 = ws + p.Q16[qc];
    MUON_LAUNCH(gemm(p, g, "Z", s));
    const float* sh = c.shift ? shift : nullptr;
    if (!fresh) {  // Q <- Q Z' + a' Q
      g = base_args(p, ws);
      set_sym(g, p, ws + p.Q16[qc], Z16, p.n_pad, snn, p.n_pad);
      g.E16 = ws + p.Q16[qc];
      g.beta_a = 1.0f;
      g.coef_a = a;
      g.shift_in = sh;
      g.out16 = ws + p.Q16[qc ^ 1];
      qc ^= 1;
      MUON_LAUNCH(gemm(p, g, "QZ", s));
    }
    fresh = false;
    if (t < c.T && ((c.restart_mask >> (t - 1)) & 1u)) {
      // restart: X <- Q X, R = X X^T, Q = I
      g = base_args(p, ws);
      set_px(g, p, ws + p.Q16[qc], ws + p.XT[xc]);
      g.out16 = ws + p.XN;
      g.outT16 = ws + p.XT[xc ^ 1];
      xc ^= 1;
      MUON_LAUNCH(gemm(p, g, "QX", s));
      MUON_LAUNCH(gram_of_x());
      fresh = true;
    } else if (t < c.T) {
      // RZ = R Z' + a' R
      g = base_args(p, ws);
      set_sym(g, p, R16, Z16, p.n_pad, snn, p.n_pad);
      g.E16 = R16;
      g.beta_a = 1.0f;
      g.coef_a = a;
      g.shift_in = sh;
      g.out16 = RZ16;
      MUON_LAUNCH(gemm(p, g, "RZ", s));
      // R <- Z' RZ + a' RZ
      g = base_args(p, ws);
      set_sym(g, p, Z16, RZ16, p.n_pad, snn, p.n_pad);
      g.E16 = RZ16;
      g.beta_a = 1.0f;
      g.coef_a = a;
      g.shift_in = sh;
      g.out16 = R16;
      g.part_out = c.shift ? tp : nullptr;
      npart = g.ntiles;
      MUON_LAUNCH(gemm(p, g, "ZRZ", s));
    }
  }
  // O = Q X
  GemmArgs g = base_args(p, ws);
  set_px(g, p, ws + p.Q16[qc], ws + p.XT[xc]);
  set_final(g, p, f);
  MUON_LAUNCH(gemm(p, g, "QX", s));
  return MUON_OK;
}

muon_status orthogonalize(muon_ns_variant v, int batch, int rows, int cols, const void* const* M,
                          muon_dtype m_dtype, void* const* O, muon_dtype o_dtype,
                          const muon_ns_config* cfg, void* workspace, size_t ws_bytes, void* stream) {
  Config c;
  muon_status st = make_config(cfg, v, &c);
  if (st != MUON_OK) return st;
  Plan p;
  if (!make_plan(batch, rows, cols, v, c, &p)) return MUON_ERR_INVALID_ARG;
  if (M == nullptr || O == nullptr) return MUON_ERR_INVALID_ARG;
  if (reinterpret_cast<const void*>(M) == reinterpret_cast<const void*>(O)) return MUON_ERR_INVALID_ARG;
  if (!valid_dtype(m_dtype)) return MUON_ERR_INVALID_ARG;
  if (o_dtype != MUON_F32 && o_dtype != MUON_BF16) return MUON_ERR_UNSUPPORTED;
  if (workspace == nullptr || ws_bytes < p.total) return MUON_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MUON_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  st = run_prologue(p, c, ws, M, m_dtype, nullptr, nullptr, 0.0, s);
  if (st != MUON_OK) return st;
  Final f{nullptr, 0, O, o_dtype, 0.0f, 0.0f, 1.0f};
  return v == MUON_NS_STANDARD ? run_standard(p, c, ws, f, s) : run_gram(p, c, ws, f, s);
}


// ---------------------------------------------------------------------------
// low-bit momentum state ([GRASP] overall framework and full example)
// ---------------------------------------------------------------------------
constexpr int kGraspMaxPieces = 8;  // k pieces of the two long power-iteration products
constexpr int kGraspMaxBatch = 65535 / kGraspMaxPieces;  // the state kernels put (batch x pieces) in grid z

int nblk(int x, int b) { return (x + b - 1) / b; }

// k pieces for a product with `tiles` output tiles and K of length `K`, each
// piece at least 256 long.  The tall products run per_cu blocks per compute
// unit (M_t Q three, M_t^T P two), and a block's time is set by its k length
// (its loads wait on memory latency, not on bandwidth shared with the others),
// so a launch of B blocks takes about ceil(B / slots) rounds of K / pieces
// each: with fewer tiles than slots, the count that minimises rounds / pieces
// is taken (the smallest on a tie, for the fewest partial sums).  Planned for
// the 256 compute units of the MI355X so that the workspace size depends on
// the shapes only.
constexpr int kGraspPlanCUs = 256;
constexpr int kMQBlocksPerCU = 3, kMtPBlocksPerCU = 2;

void grasp_pieces(int64_t tiles, int K, int per_cu, int* pieces, int* kchunk) {
  const int64_t slots = static_cast<int64_t>(kGraspPlanCUs) * per_cu;
  const int maxp = K / 256 > 1 ? (K / 256 < kGraspMaxPieces ? K / 256 : kGraspMaxPieces) : 1;
  int pcs = 1;
  if (tiles < slots) {
    double best = 0.0;
    for (int q = 1; q <= maxp; ++q) {
      const double cost = static_cast<double>((tiles * q + slots - 1) / slots) / q;
      if (q == 1 || cost < best - 1e-12) {
        best = cost;
        pcs = q;
      }
    }
  }
  int chunk = static_cast<int>(round_up(static_cast<size_t>((K + pcs - 1) / pcs), 32));
  *kchunk = chunk;
  *pieces = (K + chunk - 1) / chunk;
}

// Workspace after the Newton-Schulz part: M_t and its pointer table, then
// (k > 0) the power-iteration buffers.
struct GraspLayout {
  size_t ptrs, mt, qs, colpart, colinv, ppart, ptil, spart, S, dead, dinv, P, ps, rpart, R, total;
  int nch_n, nch_m, gchunk;
};

bool grasp_layout(size_t base, int batch, int rows, int cols, int k, GraspLayout* g) {
  memset(g, 0, sizeof(*g));
  const size_t B = static_cast<size_t>(batch), r = rows, c = cols, kk = k;
  size_t off = round_up(base, 256);
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  g->ptrs = take(B * sizeof(void*));
  g->mt = take(B * r * c * 4);
  if (k > 0) {
    g->nch_n = nblk(cols, kUnitRows);
    g->gchunk = gram_chunk_rows(rows, batch);
    g->nch_m = nblk(rows, g->gchunk);
    g->qs = take(B * c * kk * 4);  // R's codes transposed (bf16), later R split into bf16 hi and lo planes
    g->colpart = take(B * g->nch_n * kk * 8);
    g->colinv = take(B * kk * 8);
    int pcs = 1, chunk = 0;
    grasp_pieces(static_cast<int64_t>(nblk(rows, 128)) * nblk(k, 128) * batch, cols, kMQBlocksPerCU, &pcs, &chunk);
    g->ppart = take(pcs > 1 ? B * pcs * r * kk * 4 : 0);
    g->ptil = take(B * r * kk * 4);
    g->spart = take(B * g->nch_m * kk * kk * 8);
    g->S = take(B * kk * kk * 8);
    g->dead = take(B * kk * 4);
    g->dinv = take(B * nblk(k, 64) * 64 * 64 * 8);  // U's 64 x 64 diagonal blocks inverted
    g->P = take(B * r * kk * 4);
    g->ps = take(B * r * kk * 4);  // P^T split into bf16 hi and lo planes, later P
    grasp_pieces(static_cast<int64_t>(nblk(cols, 128)) * nblk(k, 128) * batch, rows, kMtPBlocksPerCU, &pcs, &chunk);
    g->rpart = take(pcs > 1 ? B * pcs * c * kk * 4 : 0);
    g->R = take(B * c * kk * 4);
  }
  g->total = off;
  return true;
}

bool grasp_state_ok(const muon_grasp_state* st, int k) {
  if (st == nullptr || st->res_codes == nullptr || st->res_row_scales == nullptr || st->res_col_scales == nullptr)
    return false;
  if (k > 0 && (st->P_codes == nullptr || st->P_scales == nullptr || st->R_codes == nullptr || st->R_scales == nullptr))
    return false;
  return true;
}

// Momentum, power iteration and the new state; M_t ends in the workspace
// (pointer table at lay.ptrs) for the Newton-Schulz part.
muon_status run_grasp_state(int batch, int rows, int cols, int k, const muon_grasp_state* st, const void* const* G,
                            int g_dtype, double mu, void* const* M_out, char* ws, const GraspLayout& lay,
                            hipStream_t s, hipStream_t s2, hipEvent_t* join) {
  const double elems = static_cast<double>(rows) * cols * batch;
  const double gsz = g_dtype == kF32 ? 4.0 : 2.0;
  float* mt = reinterpret_cast<float*>(ws + lay.mt);
  const int64_t s_mt = static_cast<int64_t>(rows) * cols;
  MUON_LAUNCH(launch_ptr_table(mt, s_mt, batch, reinterpret_cast<float**>(ws + lay.ptrs), s));
  if (k == 0) {
    GridArgs a{};
    a.rows = rows;
    a.cols = cols;
    a.codes = st->res_codes;
    a.sr = st->res_row_scales;
    a.sc = st->res_col_scales;
    a.G = G;
    a.g_dtype = g_dtype;
    a.mu = mu;
    a.Y = M_out;
    a.mt = mt;
    a.s_mt = s_mt;
    const double bytes = elems * (1.0 + gsz + 4.0 + (M_out != nullptr ? 4.0 : 0.0));
    MUON_LAUNCH(traced(s, "grid_kernel<1>", "gridq_momentum", 0.0, bytes,
                       [&] { return launch_grid(a, 1, batch, s); }));
    return MUON_OK;
  }
  const double kd = k;
  // 1. M_t = mu (deq(M_res) + deq(P) deq(R)^T) + G
  {
    ReconArgs a{};
    a.rows = rows;
    a.cols = cols;
    a.k = k;
    a.res_codes = st->res_codes;
    a.res_sr = st->res_row_scales;
    a.res_sc = st->res_col_scales;
    a.P_codes = st->P_codes;
    a.P_scales = st->P_scales;
    a.R_codes = st->R_codes;
    a.R_scales = st->R_scales;
    a.G = G;
    a.g_dtype = g_dtype;
    a.mu = mu;
    a.mt = mt;
    a.s_mt = s_mt;
    a.Y = M_out;
    const double bytes = elems * (0.5 + gsz + 4.0 + (M_out != nullptr ? 4.0 : 0.0)) + (rows + cols) * kd * batch;
    MUON_LAUNCH(traced(s, "recon_kernel", "grasp_momentum", 2.0 * elems * kd, bytes,
                       [&] { return launch_recon(a, batch, s); }));
  }
  // The rest reads M_t and the old R only: with a second stream it runs there,
  // beside Newton-Schulz on the call's stream, and joins back at the end.
  if (s2 != s) {
    hipEvent_t fork = nullptr;
    if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess) return MUON_ERR_HIP;
    const bool ok = hipEventRecord(fork, s) == hipSuccess && hipStreamWaitEvent(s2, fork, 0) == hipSuccess;
    (void)hipEventDestroy(fork);
    if (!ok) return MUON_ERR_HIP;
    s = s2;
  }
  // 2. Q = unit columns of deq(R_{t-1}), kept as R's codes and scales and the
  // column norms: the norms, and the codes transposed to bf16 (exact)
  {
    UnitArgs a{};
    a.n = cols;
    a.k = k;
    a.nchunk = lay.nch_n;
    a.codes = st->R_codes;
    a.scales = st->R_scales;
    a.part = reinterpret_cast<double*>(ws + lay.colpart);
    a.inv = reinterpret_cast<double*>(ws + lay.colinv);
    MUON_LAUNCH(traced(s, "colsq_kernel+colinv_kernel", "grasp_Q", 0.0, cols * kd * batch * 1.25,
                       [&] { return launch_col_norms(a, batch, s); }));
  }
  uint16_t* qs = reinterpret_cast<uint16_t*>(ws + lay.qs);
  const int64_t s_qs = static_cast<int64_t>(cols) * k * 2;
  MUON_LAUNCH(traced(s, "codes_t_kernel", "grasp_Q_split", 0.0, cols * kd * batch * 3.0, [&] {
    return launch_codes_t(st->R_codes, cols, k, qs, s_qs, batch, s);
  }));
  // 3. P~ = M_t Q (split along k when the tiles alone do not fill the device)
  float* ptil = reinterpret_cast<float*>(ws + lay.ptil);
  {
    MQArgs a{};
    a.M = rows;
    a.N = k;
    a.K = cols;
    a.A = mt;
    a.sA = s_mt;
    a.Ct = qs;
    a.sCt = s_qs;
    a.rs = st->R_scales;
    a.inv = reinterpret_cast<double*>(ws + lay.colinv);
    grasp_pieces(static_cast<int64_t>(nblk(rows, 128)) * nblk(k, 128) * batch, cols, kMQBlocksPerCU, &a.pieces, &a.kchunk);
    a.sC = static_cast<int64_t>(rows) * k;
    a.C = a.pieces > 1 ? reinterpret_cast<float*>(ws + lay.ppart) : ptil;
    MUON_LAUNCH(traced(s, "mq_kernel", "grasp_MQ", 2.0 * elems * kd,
                       elems * 4.0 + (cols * 2.0 + rows * 4.0 * a.pieces) * kd * batch,
                       [&] { return launch_mq(a, batch, s); }));
    if (a.pieces > 1)
      MUON_LAUNCH(traced(s, "sum_pieces_kernel", "grasp_MQ_sum", 0.0, rows * kd * batch * 4.0 * (a.pieces + 1),
                         [&] { return launch_sum_pieces(a.C, a.pieces, a.sC, ptil, batch, s); }));
  }
  // 4. CholeskyQR: S = P~^T P~ = U^T U, P = P~ U^{-1}, then its 8-bit code
  float* P = reinterpret_cast<float*>(ws + lay.P);
  {
    CholArgs a{};
    a.m = rows;
    a.k = k;
    a.nchunk = lay.nch_m;
    a.chunk = lay.gchunk;
    a.P = ptil;
    a.sP = static_cast<int64_t>(rows) * k;
    a.spart = reinterpret_cast<double*>(ws + lay.spart);
    a.S = reinterpret_cast<double*>(ws + lay.S);
    a.dead = reinterpret_cast<int*>(ws + lay.dead);
    a.Pout = P;
    a.dinv = reinterpret_cast<double*>(ws + lay.dinv);
    MUON_LAUNCH(traced(s, "gram64_kernel+gram_sum", "grasp_gram", rows * kd * kd * batch, rows * kd * 4.0 * batch,
                       [&] { return launch_gram(a, batch, s); }));
    const bool reg = k <= kRegRankK;
    MUON_LAUNCH(traced(s, reg ? "chol_reg_kernel" : "chol_panel_kernel", "grasp_cholesky", kd * kd * kd / 3.0 * batch,
                       kd * kd * 16.0 * batch, [&] { return launch_chol(a, batch, s); }));
    MUON_LAUNCH(traced(s, "row_solve_mfma_kernel", "grasp_row_solve", rows * kd * kd * batch, rows * kd * 8.0 * batch,
                       [&] { return launch_row_solve(a, batch, s); }));
    Group8Args q{};
    q.rows = rows;
    q.k = k;
    q.Xs = P;
    q.sX = a.sP;
    q.codes = st->P_codes;
    q.scales = st->P_scales;
    MUON_LAUNCH(traced(s, "group8_kernel<0>", "grasp_P_code", 0.0, rows * kd * 5.0 * batch,
                       [&] { return launch_group8(q, false, batch, s); }));
  }
  // 6. R = M_t^T P (P^T split once into bf16 planes), then its 8-bit code
  float* R = reinterpret_cast<float*>(ws + lay.R);
  uint16_t* ps = reinterpret_cast<uint16_t*>(ws + lay.ps);
  const int64_t s_ps = static_cast<int64_t>(rows) * k * 2;
  MUON_LAUNCH(traced(s, "split_t_kernel", "grasp_P_split", 0.0, rows * kd * batch * 8.0, [&] {
    return launch_split_t(P, static_cast<int64_t>(rows) * k, rows, k, ps, ps + static_cast<int64_t>(rows) * k, s_ps,
                          batch, s);
  }));
  {
    TallArgs a{};
    a.M = cols;
    a.N = k;
    a.K = rows;
    a.A = mt;
    a.sA = s_mt;
    a.a_row = 1;
    a.a_k = cols;
    a.Bh = ps;
    a.Bl = ps + static_cast<int64_t>(rows) * k;
    a.sB = s_ps;
    a.b_row = rows;
    grasp_pieces(static_cast<int64_t>(nblk(cols, 128)) * nblk(k, 128) * batch, rows, kMtPBlocksPerCU, &a.pieces, &a.kchunk);
    a.sC = static_cast<int64_t>(cols) * k;
    a.C = a.pieces > 1 ? reinterpret_cast<float*>(ws + lay.rpart) : R;
    MUON_LAUNCH(traced(s, "tall_gemm_kernel", "grasp_MtP", 2.0 * elems * kd,
                       elems * 4.0 + (rows + cols * a.pieces) * kd * 4.0 * batch,
                       [&] { return launch_tall(a, batch, s); }));
    if (a.pieces > 1)
      MUON_LAUNCH(traced(s, "sum_pieces_kernel", "grasp_MtP_sum", 0.0, cols * kd * batch * 4.0 * (a.pieces + 1),
                         [&] { return launch_sum_pieces(a.C, a.pieces, a.sC, R, batch, s); }));
    Group8Args q{};
    q.rows = cols;
    q.k = k;
    q.Xs = R;
    q.sX = a.sC;
    q.codes = st->R_codes;
    q.scales = st->R_scales;
    MUON_LAUNCH(traced(s, "group8_kernel<0>", "grasp_R_code", 0.0, cols * kd * 5.0 * batch,
                       [&] { return launch_group8(q, false, batch, s); }));
  }
  // 7. grid code of M_res = M_t - P R^T, P and R split once into bf16 planes
  // (in the buffers of R's transposed codes and of the split P^T, which M_t Q
  // and M_t^T P have used)
  {
    uint16_t* rsp = qs;
    MUON_LAUNCH(traced(s, "split_kernel", "grasp_PR_split", 0.0, (rows + cols) * kd * batch * 8.0, [&] {
      hipError_t e = launch_split(P, static_cast<int64_t>(rows) * k, static_cast<int64_t>(rows) * k, ps,
                                  ps + static_cast<int64_t>(rows) * k, s_ps, batch, s);
      if (e != hipSuccess) return e;
      return launch_split(R, static_cast<int64_t>(cols) * k, static_cast<int64_t>(cols) * k, rsp,
                          rsp + static_cast<int64_t>(cols) * k, s_qs, batch, s);
    }));
    ResidualArgs a{};
    a.rows = rows;
    a.cols = cols;
    a.prod.M = rows;
    a.prod.N = cols;
    a.prod.K = k;
    a.prod.Ah = ps;
    a.prod.Al = ps + static_cast<int64_t>(rows) * k;
    a.prod.sA = s_ps;
    a.prod.a_row = k;
    a.prod.Bh = rsp;
    a.prod.Bl = rsp + static_cast<int64_t>(cols) * k;
    a.prod.sB = s_qs;
    a.prod.b_row = k;
    a.prod.pieces = 1;
    a.prod.kchunk = k;
    a.mt = mt;
    a.s_mt = s_mt;
    a.codes = st->res_codes;
    a.sr = st->res_row_scales;
    a.sc = st->res_col_scales;
    MUON_LAUNCH(traced(s, "residual_kernel", "grasp_residual", 2.0 * elems * kd,
                       elems * 4.5 + (rows + cols) * kd * 4.0 * batch,
                       [&] { return launch_residual(a, batch, s); }));
  }
  if (join != nullptr && s == s2) {
    if (hipEventCreateWithFlags(join, hipEventDisableTiming) != hipSuccess) return MUON_ERR_HIP;
    if (hipEventRecord(*join, s2) != hipSuccess) return MUON_ERR_HIP;
  }
  return MUON_OK;
}

muon_status grasp_step(int batch, int rows, int cols, int k, void* const* W, muon_dtype w_dtype,
                       const muon_grasp_state* state, const void* const* G, muon_dtype g_dtype, float mu, float lr,
                       float weight_decay, float update_scale, muon_ns_variant variant, const muon_ns_config* cfg,
                       void* const* O_out, muon_dtype o_dtype, void* const* M_out, void* workspace,
                       size_t ws_bytes, void* stream, void* aux_stream) {
  if (variant != MUON_NS_STANDARD && variant != MUON_NS_GRAM) return MUON_ERR_INVALID_ARG;
  Config c;
  muon_status st = make_config(cfg, variant, &c);
  if (st != MUON_OK) return st;
  Plan p;
  if (!make_plan(batch, rows, cols, variant, c, &p)) return MUON_ERR_INVALID_ARG;
  const int kmax = rows < cols ? rows : cols;
  if (k < 0 || k > kmax || k > MUON_GRASP_MAX_K) return MUON_ERR_INVALID_ARG;
  if (W == nullptr || G == nullptr || !grasp_state_ok(state, k)) return MUON_ERR_INVALID_ARG;
  if (batch > kGraspMaxBatch) return MUON_ERR_INVALID_ARG;
  {
    const void* arrays[4] = {W, G, O_out, M_out};
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (arrays[i] != nullptr && arrays[i] == arrays[j]) return MUON_ERR_INVALID_ARG;
  }
  if (!isfinite(mu) || !isfinite(lr) || !isfinite(weight_decay) || !isfinite(update_scale)) return MUON_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype) || !valid_dtype(g_dtype)) return MUON_ERR_INVALID_ARG;
  if (w_dtype == MUON_F16) return MUON_ERR_UNSUPPORTED;
  if (O_out != nullptr && o_dtype != MUON_F32 && o_dtype != MUON_BF16) return MUON_ERR_UNSUPPORTED;
  GraspLayout lay;
  grasp_layout(p.total, batch, rows, cols, k, &lay);
  if (workspace == nullptr || ws_bytes < lay.total) return MUON_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MUON_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipStream_t s2 = aux_stream != nullptr && k > 0 ? static_cast<hipStream_t>(aux_stream) : s;
  hipEvent_t join = nullptr;
  st = run_grasp_state(batch, rows, cols, k, state, G, g_dtype, static_cast<double>(mu), M_out, ws, lay, s, s2,
                       s2 != s ? &join : nullptr);
  if (st == MUON_OK)
    st = run_prologue(p, c, ws, reinterpret_cast<const void* const*>(ws + lay.ptrs), kF32, nullptr, nullptr, 0.0, s);
  if (st == MUON_OK) {
    Final f{W, w_dtype, O_out, o_dtype, lr, weight_decay, update_scale};
    st = variant == MUON_NS_STANDARD ? run_standard(p, c, ws, f, s) : run_gram(p, c, ws, f, s);
  }
  if (join != nullptr) {  // the call ends on `stream` with the state update done
    if (hipStreamWaitEvent(s, join, 0) != hipSuccess && st == MUON_OK) st = MUON_ERR_HIP;
    (void)hipEventDestroy(join);
  }
  return st;
}

muon_status grid_codec(int mode, int batch, int rows, int cols, const void* const* X, void* const* codes,
                       void* const* sr, void* const* sc, void* const* Y, void* stream) {
  if (batch < 1 || rows < 1 || cols < 1 || rows > MUON_MAX_DIM || cols > MUON_MAX_DIM) return MUON_ERR_INVALID_ARG;
  if (batch > 65535) return MUON_ERR_INVALID_ARG;
  if (codes == nullptr || sr == nullptr || sc == nullptr) return MUON_ERR_INVALID_ARG;
  if ((mode == 0 && X == nullptr) || (mode == 2 && Y == nullptr)) return MUON_ERR_INVALID_ARG;
  GridArgs a{};
  a.rows = rows;
  a.cols = cols;
  a.X = X;
  a.codes = codes;
  a.sr = sr;
  a.sc = sc;
  a.Y = Y;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double elems = static_cast<double>(rows) * cols * batch;
  MUON_LAUNCH(traced(s, mode == 0 ? "grid_kernel<0>" : "grid_kernel<2>", mode == 0 ? "grid_quantize" : "grid_dequantize",
                     0.0, elems * 4.5, [&] { return launch_grid(a, mode, batch, s); }));
  return MUON_OK;
}

muon_status group8_codec(bool dequantize, int batch, int rows, int k, void* const* X, void* const* codes,
                         void* const* scales, void* stream) {
  if (batch < 1 || rows < 1 || k < 1 || rows > MUON_MAX_DIM || k > MUON_MAX_DIM) return MUON_ERR_INVALID_ARG;
  if (batch > 65535) return MUON_ERR_INVALID_ARG;
  if (X == nullptr || codes == nullptr || scales == nullptr) return MUON_ERR_INVALID_ARG;
  Group8Args a{};
  a.rows = rows;
  a.k = k;
  a.Xp = X;
  a.codes = codes;
  a.scales = scales;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MUON_LAUNCH(traced(s, dequantize ? "group8_kernel<1>" : "group8_kernel<0>",
                     dequantize ? "group8_dequantize" : "group8_quantize", 0.0,
                     static_cast<double>(rows) * k * batch * 5.0, [&] { return launch_group8(a, dequantize, batch, s); }));
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// The step, with the caller's workspace or the fixed device scratch below.
// ---------------------------------------------------------------------------
}  // namespace

// Scratch memory of muon_step_fixed_scratch, for callers that cannot
// allocate: one copy per device, held until the process ends.  Host code
// never uses this name as an address; it takes the device address from
// hipGetSymbolAddress once per device (scratch_address below).
static __device__ __align__(256) char scratch[MUON_FIXED_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call there; null if the lookup fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

muon_status step(int batch, int rows, int cols, void* const* W, muon_dtype w_dtype, void* const* M,
                 const void* const* G, muon_dtype state_dtype, float mu, float lr, float weight_decay,
                 float update_scale, muon_ns_variant variant, const muon_ns_config* cfg, void* const* O_out,
                 muon_dtype o_dtype, void* workspace, size_t ws_bytes, void* stream, bool fixed_scratch) {
  if (variant != MUON_NS_STANDARD && variant != MUON_NS_GRAM) return MUON_ERR_INVALID_ARG;
  Config c;
  muon_status st = make_config(cfg, variant, &c);
  if (st != MUON_OK) return st;
  Plan p;
  if (!make_plan(batch, rows, cols, variant, c, &p)) return MUON_ERR_INVALID_ARG;
  if (W == nullptr || M == nullptr || G == nullptr) return MUON_ERR_INVALID_ARG;
  const void* arrays[4] = {W, M, G, O_out};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (arrays[i] != nullptr && arrays[i] == arrays[j]) return MUON_ERR_INVALID_ARG;
  if (!isfinite(mu) || !isfinite(lr) || !isfinite(weight_decay) || !isfinite(update_scale)) return MUON_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype) || !valid_dtype(state_dtype)) return MUON_ERR_INVALID_ARG;
  if (w_dtype == MUON_F16 || state_dtype == MUON_F16) return MUON_ERR_UNSUPPORTED;
  if (O_out != nullptr && o_dtype != MUON_F32 && o_dtype != MUON_BF16) return MUON_ERR_UNSUPPORTED;
  if (fixed_scratch) {  // every check above passed: only now touch the device
    if (p.total > MUON_FIXED_SCRATCH_BYTES) return MUON_ERR_WORKSPACE;
    workspace = scratch_address();
    if (workspace == nullptr) return MUON_ERR_HIP;
    ws_bytes = MUON_FIXED_SCRATCH_BYTES;
  }
  if (workspace == nullptr || ws_bytes < p.total) return MUON_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MUON_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  st = run_prologue(p, c, ws, reinterpret_cast<const void* const*>(M), state_dtype, G, M,
                    static_cast<double>(mu), s);
  if (st != MUON_OK) return st;
  Final f{W, w_dtype, O_out, o_dtype, lr, weight_decay, update_scale};
  return variant == MUON_NS_STANDARD ? run_standard(p, c, ws, f, s) : run_gram(p, c, ws, f, s);
}

}  // namespace

extern "C" {

void muon_ns_config_init(muon_ns_config* cfg, muon_ns_variant variant) {
  if (cfg == nullptr) return;
  cfg->T = 5;
  cfg->coeffs = nullptr;
  cfg->eps = 1e-7f;
  cfg->restart_mask = variant == MUON_NS_GRAM ? (1u << 1) : 0u;
  cfg->compute = variant == MUON_NS_GRAM ? MUON_F16 : MUON_BF16;
  cfg->shift = 1;
}

size_t muon_workspace_size(int batch, int rows, int cols, muon_ns_variant variant,
                           const muon_ns_config* cfg) {
  Config c;
  if (make_config(cfg, variant, &c) != MUON_OK) return 0;
  Plan p;
  if (!make_plan(batch, rows, cols, variant, c, &p)) return 0;
  return p.total;
}

muon_status ns_orthogonalize(int batch, int rows, int cols, const void* const* M, muon_dtype m_dtype,
                             void* const* O, muon_dtype o_dtype, const muon_ns_config* cfg,
                             void* workspace, size_t ws_bytes, void* stream) {
  return orthogonalize(MUON_NS_STANDARD, batch, rows, cols, M, m_dtype, O, o_dtype, cfg, workspace,
                       ws_bytes, stream);
}

muon_status gram_ns_orthogonalize(int batch, int rows, int cols, const void* const* M,
                                  muon_dtype m_dtype, void* const* O, muon_dtype o_dtype,
                                  const muon_ns_config* cfg, void* workspace, size_t ws_bytes,
                                  void* stream) {
  return orthogonalize(MUON_NS_GRAM, batch, rows, cols, M, m_dtype, O, o_dtype, cfg, workspace,
                       ws_bytes, stream);
}

muon_status muon_step(int batch, int rows, int cols, void* const* W, muon_dtype w_dtype, void* const* M,
                      const void* const* G, muon_dtype state_dtype, float mu, float lr,
                      float weight_decay, float update_scale, muon_ns_variant variant, const muon_ns_config* cfg,
                      void* const* O_out, muon_dtype o_dtype, void* workspace, size_t ws_bytes,
                      void* stream) {
  return step(batch, rows, cols, W, w_dtype, M, G, state_dtype, mu, lr, weight_decay, update_scale, variant, cfg,
              O_out, o_dtype, workspace, ws_bytes, stream, false);
}

muon_status muon_step_fixed_scratch(int batch, int rows, int cols, void* const* W, muon_dtype w_dtype,
                                    void* const* M, const void* const* G, muon_dtype state_dtype, float mu,
                                    float lr, float weight_decay, float update_scale, muon_ns_variant variant,
                                    const muon_ns_config* cfg, void* const* O_out, muon_dtype o_dtype,
                                    void* stream) {
  return step(batch, rows, cols, W, w_dtype, M, G, state_dtype, mu, lr, weight_decay, update_scale, variant, cfg,
              O_out, o_dtype, nullptr, 0, stream, true);
}

size_t muon_grasp_workspace_size(int batch, int rows, int cols, int k, muon_ns_variant variant,
                                 const muon_ns_config* cfg) {
  Config c;
  if (make_config(cfg, variant, &c) != MUON_OK) return 0;
  Plan p;
  if (!make_plan(batch, rows, cols, variant, c, &p)) return 0;
  const int kmax = rows < cols ? rows : cols;
  if (k < 0 || k > kmax || k > MUON_GRASP_MAX_K) return 0;
  GraspLayout lay;
  grasp_layout(p.total, batch, rows, cols, k, &lay);
  return lay.total;
}

muon_status muon_grasp_step(int batch, int rows, int cols, int k, void* const* W, muon_dtype w_dtype,
                            const muon_grasp_state* state, const void* const* G, muon_dtype g_dtype, float mu,
                            float lr, float weight_decay, float update_scale, muon_ns_variant variant,
                            const muon_ns_config* cfg, void* const* O_out, muon_dtype o_dtype, void* const* M_out,
                            void* workspace, size_t ws_bytes, void* stream, void* aux_stream) {
  return grasp_step(batch, rows, cols, k, W, w_dtype, state, G, g_dtype, mu, lr, weight_decay, update_scale, variant,
                    cfg, O_out, o_dtype, M_out, workspace, ws_bytes, stream, aux_stream);
}

muon_status muon_grid_quantize(int batch, int rows, int cols, const void* const* X, void* const* codes,
                               void* const* row_scales, void* const* col_scales, void* stream) {
  return grid_codec(0, batch, rows, cols, X, codes, row_scales, col_scales, nullptr, stream);
}

muon_status muon_grid_dequantize(int batch, int rows, int cols, const void* const* codes,
                                 const void* const* row_scales, const void* const* col_scales, void* const* Y,
                                 void* stream) {
  return grid_codec(2, batch, rows, cols, nullptr, const_cast<void* const*>(codes),
                    const_cast<void* const*>(row_scales), const_cast<void* const*>(col_scales), Y, stream);
}

muon_status muon_group8_quantize(int batch, int rows, int k, const void* const* X, void* const* codes,
                                 void* const* scales, void* stream) {
  return group8_codec(false, batch, rows, k, const_cast<void* const*>(X), codes, scales, stream);
}

muon_status muon_group8_dequantize(int batch, int rows, int k, const void* const* codes, const void* const* scales,
                                   void* const* Y, void* stream) {
  return group8_codec(true, batch, rows, k, Y, const_cast<void* const*>(codes), const_cast<void* const*>(scales),
                      stream);
}

double muon_ns_flops(int rows, int cols, muon_ns_variant variant, const muon_ns_config* cfg,
                     int symmetric_aware) {
  Config c;
  if (make_config(cfg, variant, &c) != MUON_OK) return 0.0;
  if (rows < 1 || cols < 1) return 0.0;
  const double n = rows < cols ? rows : cols;
  const double m = rows < cols ? cols : rows;
  const double n3 = n * n * n, mn2 = m * n * n;
  const double T = c.T;
  const double k = symmetric_aware ? 1.0 : 2.0;  // cost of a symmetric product relative to n^3 / m n^2
  if (variant == MUON_NS_STANDARD) {
    // per iteration: X X^T (m n^2, symmetric), A A (n^3, symmetric), B X (2 m n^2)
    return T * (k * mn2 + k * n3 + 2.0 * mn2);
  }
  int r = 0;
  for (int t = 1; t < c.T; ++t) r += (c.restart_mask >> (t - 1)) & 1u;
  // R R every iteration; Q Z except when Q is fresh (t = 1 and after each
  // restart); R Z and Z (RZ) for t < T without a restart; X X^T and Q X once
  // plus once per restart.
  const double rr = T, qz = T - 1 - r, upd = 2.0 * (T - 1 - r), sy = 1 + r, qx = 1 + r;
  return k * (rr + qz + upd) * n3 + (k * sy + 2.0 * qx) * mn2;
}

const char* muon_status_string(muon_status status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_UNSUPPORTED: return "unsupported dtype combination";
    case MUON_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MUON_ERR_HIP: return "HIP launch failed";
    default: break;
  }
  return "unknown status";
}

int muon_abi_version(void) { return MUON_ABI_VERSION; }

int muon_trace_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_trace.mu);
  const int prev = g_trace.on ? 1 : 0;
  for (TraceRec& r : g_trace.recs) {
    g_trace.pool.push_back(r.e0);
    g_trace.pool.push_back(r.e1);
  }
  g_trace.recs.clear();
  g_trace.on = enable != 0;
  return prev;
}

int muon_trace_collect(muon_trace_record* out, int max) {
  std::lock_guard<std::mutex> lock(g_trace.mu);
  int failed = 0;
  const int count = static_cast<int>(g_trace.recs.size());
  for (int i = 0; i < count; ++i) {
    TraceRec& r = g_trace.recs[i];
    float ms = 0.0f;
    if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) failed = 1;
    r.rec.ms = ms;
    if (out != nullptr && i < max) out[i] = r.rec;
    g_trace.pool.push_back(r.e0);
    g_trace.pool.push_back(r.e1);
  }
  g_trace.recs.clear();
  return failed ? -1 : count;
}

}  // extern "C"
