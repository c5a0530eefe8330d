"""fp64 CPU oracle for the low-bit momentum state of 4-bit-Muon-GRASP
(test infrastructure only).

Only the test suite may import this module; the library never does, and the
two share no code.  Plain numpy, slow and obvious on purpose.

Source: notes on "Achieving low-bit Muon through subspace preservation and
grid quantization" (ICLR 2026), cited as [GRASP]:

* overall framework and the full example: per step, dequantise the stored
  residual (4 bit) and top-subspace factors P, R (8 bit), rebuild
  M_{t-1} = M_res + P R^T, take Q = R with unit columns, form
  M_t = mu M_{t-1} + G, one power-iteration step P <- M_t Q, orthonormalise
  P by QR, R <- M_t^T P, store M_res = M_t - P R^T in 4 bit (grid) and P, R in
  8 bit; Newton-Schulz runs on the full M_t and W <- W - lr (O + wd W);
* key design 1: the top subspace, rank k (default: 1/16 of the rank);
* key design 2: grid quantisation over s x s blocks (s = 128) with a scale per
  row and per column of each block and x / min(row scale, column scale);
* training strategy: INT4 / INT8 formats, group and grid size 128.

Readings where the page is silent (each also in the design notes):

G1  "largest entry" of a block row or column is the largest magnitude (a
    symmetric quantiser), NaN propagating.
G2  4-bit codes are the integers -7..7.  Encoding: q = rint(7 x / m) with
    m = min(row scale, column scale), evaluated in fp64 from the fp32 value x
    and the fp32 scales (7 x is exact there), ties to even; m = 0 or m not
    finite gives q = 0.  |x| <= m, so |q| <= 7 without clamping.  Decoding:
    x^ = q m / 7 in fp64.
G3  Storage: 4-bit codes two per byte along a row (even column in the low
    nibble, two's complement); row scales [rows][ceil(cols/128)] and column
    scales [ceil(rows/128)][cols], fp32.  Edge blocks cover the real rows and
    columns only.
G4  8-bit group quantisation of P (m x k) and R (n x k): each row is cut into
    groups of 128 consecutive entries (the last one shorter); scale = largest
    magnitude of the group (fp32); q = rint(127 x / scale) in fp64 from the
    fp32 value (codes -127..127); x^ = q scale / 127 in fp64.
G5  M_t = mu M_{t-1} + G is evaluated in fp64 (product and sum rounded in
    fp64 separately) and rounded once to fp32; the power iteration, the
    residual and Newton-Schulz all read this fp32 M_t.
G6  "QR orthogonalisation" is the Q factor with a positive diagonal in the
    triangular factor (unique for full column rank), i.e. Gram-Schmidt in
    column order; a column whose part orthogonal to the earlier columns has
    squared norm <= 1e-12 of its own squared norm (or is zero) is set to zero.
    Columns of R_{t-1} with zero norm stay zero in Q.
G7  P_t and R_t enter the residual at full precision (M_res = M_t - P_t R_t^T
    with the power-iteration factors, rounded to fp32 before quantisation);
    the 8-bit codes are made from P_t and R_t rounded to fp32.
G8  The first step starts from a caller-provided state: residual and P zero,
    R any n x k matrix (e.g. a quantised Gaussian), so that M_{-1} = 0 and
    the power iteration has a start.  k = 0 is the grid-quantised momentum
    without a subspace (the notes' "directly compress the momentum" control).
"""
from __future__ import annotations

import numpy as np

from oracle import muon_oracle as mo

S = 128        # grid block edge and group size
L4 = 7         # largest 4-bit code magnitude
L8 = 127       # largest 8-bit code magnitude
DEP_TOL = 1e-12  # G6: squared-norm ratio below which a column counts as dependent


def _nblocks(n):
    return (n + S - 1) // S


def _absmax(a, axis):
    """Largest magnitude along ``axis``, NaN propagating (G1)."""
    return np.max(np.abs(a), axis=axis) if a.shape[axis] else np.zeros(a.shape[1 - axis], a.dtype)


# --------------------------------------------------------------------------
# 4-bit grid quantisation ([GRASP] key design 2)
# --------------------------------------------------------------------------
def grid_scales(x):
    """Row scales [rows][ceil(cols/128)] and column scales [ceil(rows/128)][cols]."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    sr = np.zeros((rows, _nblocks(cols)), dtype=np.float32)
    sc = np.zeros((_nblocks(rows), cols), dtype=np.float32)
    for bc in range(_nblocks(cols)):
        sr[:, bc] = _absmax(x[:, bc * S:(bc + 1) * S], 1)
    for br in range(_nblocks(rows)):
        sc[br, :] = _absmax(x[br * S:(br + 1) * S, :], 0)
    return sr, sc


def grid_min_scale(sr, sc, rows, cols):
    """m[i, j] = min(scale of row i in j's block, scale of column j in i's block)."""
    r = np.repeat(np.asarray(sr, np.float32), S, axis=1)[:, :cols]
    c = np.repeat(np.asarray(sc, np.float32), S, axis=0)[:rows, :]
    return np.minimum(r, c)


def _encode(x, m, levels):
    x = np.asarray(x, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    ok = (m > 0) & np.isfinite(m)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(ok, (levels * x) / np.where(ok, m, 1.0), 0.0)
    return np.rint(t).astype(np.int32)


def grid_quantize(x):
    """(codes int8 in -7..7, row scales, column scales) of an fp32 matrix (G2)."""
    x = np.asarray(x, dtype=np.float32)
    sr, sc = grid_scales(x)
    q = _encode(x, grid_min_scale(sr, sc, *x.shape), L4).astype(np.int8)
    return q, sr, sc


def grid_dequantize(q, sr, sc):
    """fp64 values q m / 7 (G2)."""
    q = np.asarray(q)
    m = grid_min_scale(sr, sc, *q.shape).astype(np.float64)
    return (q.astype(np.float64) * m) / L4


def pack_nibbles(q):
    """Two 4-bit codes per byte along each row, even column low (G3)."""
    q = np.asarray(q, dtype=np.int8)
    rows, cols = q.shape
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    if cols % 2:
        u = np.concatenate([u, np.zeros((rows, 1), dtype=np.uint8)], axis=1)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b, cols):
    b = np.asarray(b, dtype=np.uint8)
    q = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int8)
    for half, shift in ((0, 0), (1, 4)):
        v = ((b >> shift) & 0xF).astype(np.int16)
        q[:, half::2] = np.where(v > 7, v - 16, v).astype(np.int8)
    return q[:, :cols]


# --------------------------------------------------------------------------
# 8-bit group quantisation of P and R ([GRASP] training strategy, G4)
# --------------------------------------------------------------------------
def group8_quantize(x):
    """(codes int8 in -127..127, scales [rows][ceil(k/128)]) of an fp32 matrix."""
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    s = np.zeros((rows, _nblocks(k)), dtype=np.float32)
    for g in range(_nblocks(k)):
        s[:, g] = _absmax(x[:, g * S:(g + 1) * S], 1)
    m = np.repeat(s, S, axis=1)[:, :k]
    return _encode(x, m, L8).astype(np.int8), s


def group8_dequantize(q, s):
    q = np.asarray(q)
    m = np.repeat(np.asarray(s, np.float64), S, axis=1)[:, :q.shape[1]]
    return (q.astype(np.float64) * m) / L8


# --------------------------------------------------------------------------
# power iteration ([GRASP] key design 1 and the full example)
# --------------------------------------------------------------------------
def orthonormalize_columns(P):
    """Q factor of QR with positive diagonal, by Gram-Schmidt in column order
    (G6); dependent or zero columns become zero."""
    P = np.asarray(P, dtype=np.float64)
    out = np.zeros_like(P)
    for j in range(P.shape[1]):
        p = P[:, j]
        v = p.copy()
        for _ in range(2):  # re-orthogonalise once: the fp64 Q factor to rounding level
            for l in range(j):
                v -= out[:, l] * (out[:, l] @ v)
        nv, np_ = v @ v, p @ p
        if np_ > 0 and nv > DEP_TOL * np_:
            out[:, j] = v / np.sqrt(nv)
    return out


def unit_columns(R):
    """Q_t: the columns of R_{t-1} scaled to unit norm (zero columns stay zero)."""
    R = np.asarray(R, dtype=np.float64)
    nrm = np.sqrt((R * R).sum(axis=0))
    return np.where(nrm > 0, R / np.where(nrm > 0, nrm, 1.0), 0.0)


def power_iteration(M, R_prev):
    """One warm-started step: Q = unit columns of R_prev, P = orth(M Q),
    R = M^T P.  Returns (P, R) in fp64; P R^T approximates the top-k part."""
    M = np.asarray(M, dtype=np.float64)
    P = orthonormalize_columns(M @ unit_columns(R_prev))
    return P, M.T @ P


# --------------------------------------------------------------------------
# the step on the low-bit state ([GRASP] overall framework, full example)
# --------------------------------------------------------------------------
def new_state(rows, cols, k, R_init=None):
    """The state before the first step (G8): zero residual and P; R from the
    caller (its 8-bit codes), or none when k = 0."""
    st = dict(res_codes=np.zeros((rows, cols), np.int8),
              res_sr=np.zeros((rows, _nblocks(cols)), np.float32),
              res_sc=np.zeros((_nblocks(rows), cols), np.float32))
    if k > 0:
        st["P_codes"] = np.zeros((rows, k), np.int8)
        st["P_scales"] = np.zeros((rows, _nblocks(k)), np.float32)
        st["R_codes"], st["R_scales"] = group8_quantize(np.asarray(R_init, np.float32))
    return st


def reconstruct(state):
    """M_{t-1} = M_res + P R^T from the stored codes (fp64)."""
    M = grid_dequantize(state["res_codes"], state["res_sr"], state["res_sc"])
    if "P_codes" in state:
        P = group8_dequantize(state["P_codes"], state["P_scales"])
        R = group8_dequantize(state["R_codes"], state["R_scales"])
        M = M + P @ R.T
    return M


def momentum(state, G, mu):
    """M_t (fp32 values, as fp64) per G5."""
    M_prev = reconstruct(state)
    return (np.float64(mu) * M_prev + np.asarray(G, np.float64)).astype(np.float32).astype(np.float64)


def compress(M_t, state):
    """New state from M_t: power iteration (k > 0), residual, quantisation.
    Returns (new_state, details) where details holds P, R (fp64) and M_res
    (fp32 values) for inspection."""
    out = {}
    det = {}
    if "P_codes" in state:
        R_prev = group8_dequantize(state["R_codes"], state["R_scales"])
        P, R = power_iteration(M_t, R_prev)
        res = (M_t - P @ R.T).astype(np.float32)
        out["P_codes"], out["P_scales"] = group8_quantize(P.astype(np.float32))
        out["R_codes"], out["R_scales"] = group8_quantize(R.astype(np.float32))
        det["P"], det["R"] = P, R
    else:
        res = np.asarray(M_t, np.float32)
    out["res_codes"], out["res_sr"], out["res_sc"] = grid_quantize(res)
    det["M_res"] = res.astype(np.float64)
    return out, det


def grasp_step(W, state, G, mu, lr, weight_decay=0.0, variant="standard", coeffs=None, T=5,
               eps=mo.EPS, restarts=(2,), update_scale=1.0, w_dtype="f32"):
    """One Muon step whose momentum lives in the low-bit state.  Returns
    (W_new, new_state, O, M_t, details).  O = NS(M_t) on the full M_t."""
    M_t = momentum(state, G, mu)
    st, det = compress(M_t, state)
    if variant == "standard":
        O = mo.newton_schulz(M_t, coeffs, T, eps)
    else:
        O = mo.gram_newton_schulz(M_t, coeffs, T, eps, restarts)
    W = np.asarray(W, np.float64)
    W_new = mo.round_to(W - lr * (update_scale * O + weight_decay * W), w_dtype)
    return W_new, st, O, M_t, det
