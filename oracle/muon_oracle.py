"""fp64 CPU oracle for the Muon step (test infrastructure only).

This module is the reference that the HIP path is checked against.  It is
test infrastructure: only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the library never does.  It
shares no code with the GPU path.  Everything is plain numpy in float64,
written from the pages, slow and obvious on purpose: matrix products are
numpy ``@`` and nothing is blocked, fused or reordered.

Sources (cited by short name):

* [GNS]     "优化器 (3)（Gram Newton-Schulz）", blog notes on Gram
            Newton-Schulz (phycat-blog).  Authority for the iteration.
* [GRASP]   notes on "Achieving low-bit Muon through subspace preservation
            and grid quantization" (ICLR 2026), section on the overall
            framework: the standard Muon step.
* [LiMuon]  notes on LiMuon (arXiv 2509.14562), design 3: the quintic
            coefficients (3.4445, -4.7750, 2.0315).
* [MuonBlog] "Muon Optimizer" blog post, section 1: momentum form; Muon is
            applied to 2-D matrices only; section 5 item 4: weight decay and a
            per-parameter update scale (no formula given: a plain factor on O).

Readings where the pages are silent or garbled (each also listed in the
design notes of the repository):

* The display equations of [GNS] are lost in extraction.  Eq.(2) is
  rebuilt from the three products listed under it in [GNS §1.2]:
  A = X X^T, B = b A + c A^2, X <- a X + B X.
* The loop ranges of [GNS §3.4 Alg.2] are lost; the restart comes after
  iteration 2 ([GNS §3.2]), so the loops are t = 1..2 and t = 3..5.
  ``restarts`` generalises this: a restart after iteration t for every t in
  the set (t < T).  The empty set is Alg.1 ([GNS §2.3]).
* Orientation: [GNS §1.2] assumes n <= m for an n x m matrix; a matrix with
  more rows than columns is iterated transposed and the result transposed
  back.
* Normalisation: X0 = X / (||X||_F + eps), eps = 1e-7 ([GNS §2.3 Alg.1]).
* Momentum: heavy ball M_t = mu M_{t-1} + G_t with M_0 = 0 ([GRASP
  framework], [GNS §1.1 eq.(1)], [MuonBlog §1]); no Nesterov term.  The new
  momentum is rounded (round to nearest even) to the state dtype and the
  iteration consumes the rounded value.
* Update: W_t = W_{t-1} - lr (O_t + wd W_{t-1}) ([GRASP] full example adds
  the wd term; wd = 0 gives the plain update), rounded to the weight dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# [LiMuon design 3]: p(z) = 3.4445 - 4.7750 z + 2.0315 z^2 used for every t.
QUINTIC = (3.4445, -4.7750, 2.0315)
EPS = 1e-7  # [GNS §2.3 Alg.1]


# --------------------------------------------------------------------------
# storage rounding (round to nearest, ties to even) from exact float64 values
# --------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, fp32 exponent
    range), ties to even, returned as float64.  Done directly on the float64
    bit pattern so there is exactly one rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)  # ravel() below must be a view
    out = np.empty_like(x)
    flat = x.ravel()
    o = out.ravel()
    bits = flat.view(np.uint64)
    expo = ((bits >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    # normal bf16 range: unbiased exponent >= -126
    normal = (expo - 1023) >= -126
    finite = expo != 0x7FF
    sel = normal & finite
    b = bits[sel]
    low = b & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    keep = b >> np.uint64(45)
    up = (low > half) | ((low == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    keep = keep + up.astype(np.uint64)
    o[sel] = (keep << np.uint64(45)).view(np.float64)
    # below the normal range: fixed absolute quantum 2^-133
    small = (~normal) & finite
    q = 2.0 ** -133
    o[small] = np.round(flat[small] / q) * q  # np.round is half-to-even
    o[~finite] = flat[~finite]
    # values that rounded past the largest bf16 become infinities
    big = np.abs(o) > 3.3895313892515355e38
    o[big] = np.copysign(np.inf, o[big])
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to a storage dtype ('f64', 'f32', 'bf16', 'f16')."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# FLOP bookkeeping ([GNS §1.2], [GNS §2.4], [GNS §3.4])
# --------------------------------------------------------------------------
@dataclass
class FlopCounter:
    """Counts the products an implementation following the pages performs.

    ``dense`` adds 2*r*K*c per product.  ``symmetric`` adds half of that for
    a product whose result is symmetric in exact arithmetic (only one
    triangle is computed, [GNS §2.4]) and the full amount otherwise.
    Products with an identity operand are free ([GNS §2.4]: Q_1 = Z_1)."""

    dense: int = 0
    symmetric: int = 0
    gemms: int = 0
    log: list = field(default_factory=list)

    def add(self, name: str, r: int, k: int, c: int, sym_result: bool):
        d = 2 * r * k * c
        self.dense += d
        self.symmetric += d // 2 if sym_result else d
        self.gemms += 1
        self.log.append((name, r, k, c, sym_result))


def _mm(P, Q, counter, name, sym_result):
    if counter is not None:
        counter.add(name, P.shape[0], P.shape[1], Q.shape[1], sym_result)
    return P @ Q


def _coeff_table(coeffs, T):
    if coeffs is None:
        return [QUINTIC] * T
    coeffs = [tuple(float(v) for v in c) for c in coeffs]
    if len(coeffs) != T:
        raise ValueError("need one (a, b, c) triple per iteration")
    return coeffs


def _orient(M):
    """[GNS §1.2]: work on the n x m orientation with n <= m."""
    M = np.asarray(M, dtype=np.float64)
    if M.ndim != 2:
        raise ValueError("the Muon step is defined for 2-D matrices")
    if M.shape[0] > M.shape[1]:
        return M.T, True
    return M, False


# --------------------------------------------------------------------------
# standard Newton-Schulz ([GNS §1.2 eq.(2)])
# --------------------------------------------------------------------------
def newton_schulz(M, coeffs=None, T=5, eps=EPS, counter=None):
    """Standard quintic Newton-Schulz: X <- a_t X + (b_t A + c_t A^2) X with
    A = X X^T, from X0 = X / (||X||_F + eps), for t = 1..T."""
    X, transposed = _orient(M)
    table = _coeff_table(coeffs, T)
    X = X / (np.linalg.norm(X) + eps)
    for (a, b, c) in table:
        A = _mm(X, X.T, counter, "XXt", True)
        A2 = _mm(A, A, counter, "A2", True)
        B = b * A + c * A2
        X = a * X + _mm(B, X, counter, "BX", False)
    return X.T if transposed else X


# --------------------------------------------------------------------------
# Gram Newton-Schulz ([GNS §2.3 Alg.1], [GNS §3.4 Alg.2])
# --------------------------------------------------------------------------
def gram_newton_schulz(M, coeffs=None, T=5, eps=EPS, restarts=(2,), counter=None,
                       R0=None, trace=None, gram_round=None):
    """Gram Newton-Schulz with restarts.

    R = X X^T, Q = I; for t = 1..T: Z = b R + c R^2; Q <- Q Z + a Q; then
    either restart (X <- Q X, R = X X^T, Q = I) when t is in ``restarts`` and
    t < T, or update R: RZ = R Z + a R; R <- Z RZ + a RZ (skipped at t = T,
    whose R is never used).  Return Q X.

    ``R0`` replaces the initial Gram matrix (used to study a spurious negative
    eigenvalue, [GNS §3.1 Prop.2]); ``trace`` (a list) receives (t, R, Q_t)
    after every iteration t for inspection: R as it stands after the
    iteration (the new Gram matrix after a restart) and Q_t as updated in
    iteration t, before a restart resets it.  ``gram_round`` ('bf16' or
    'f16') rounds every Gram matrix X X^T the iteration forms (the initial
    one and each restart's) to that type, as a 16-bit Gram product stores it
    ([GNS §3.1]: this rounding gives R_0 small negative eigenvalues); None
    keeps them exact."""
    X, transposed = _orient(M)
    n = X.shape[0]
    table = _coeff_table(coeffs, T)
    restarts = set(int(t) for t in restarts)
    X = X / (np.linalg.norm(X) + eps)
    I = np.eye(n)

    def gram(Y):
        G = _mm(Y, Y.T, counter, "XXt", True)
        return G if gram_round is None else round_to(G, gram_round)

    R = gram(X) if R0 is None else np.array(R0, dtype=np.float64)
    Q = I
    fresh = True  # Q is the identity: the product Q Z needs no GEMM
    for t, (a, b, c) in enumerate(table, start=1):
        Z = b * R + c * _mm(R, R, counter, "R2", True)
        if fresh:
            Q = Q @ Z + a * Q  # identity operand: exact, no FLOPs counted
        else:
            Q = _mm(Q, Z, counter, "QZ", True) + a * Q
        fresh = False
        Q_t = Q
        if t < T and t in restarts:
            X = _mm(Q, X, counter, "QX", False)
            R = gram(X)
            Q = I
            fresh = True
        elif t < T:
            RZ = _mm(R, Z, counter, "RZ", True) + a * R
            R = _mm(Z, RZ, counter, "ZRZ", True) + a * RZ
        if trace is not None:
            trace.append((t, R.copy(), Q_t.copy()))
    O = _mm(Q, X, counter, "QX", False)
    return O.T if transposed else O


def restart_diagnostics(M, coeffs=None, T=5, restarts=(2,), eps=EPS, gram_round=None, R0=None):
    """The two quantities [GNS §3.2] judges a restart point by: the smallest
    eigenvalue of every Gram matrix R the iteration forms (R_0, the R_t it
    updates, and each restart's new X X^T; R at t = T is never formed) and
    the condition number (largest over smallest singular value) of Q_t after
    each iteration t = 1..T.  Gram matrices are rounded as ``gram_round``
    says (see gram_newton_schulz); ``R0`` replaces the initial one (e.g. with
    a spurious negative eigenvalue, [GNS §3.1]).  Returns (lambda_min list,
    cond list)."""
    if R0 is None:
        X, _ = _orient(M)
        X = X / (np.linalg.norm(X) + eps)
        R0 = X @ X.T
        if gram_round is not None:
            R0 = round_to(R0, gram_round)
    R0 = np.array(R0, dtype=np.float64)
    trace = []
    gram_newton_schulz(M, coeffs, T, eps, restarts, R0=R0, trace=trace, gram_round=gram_round)
    lam = [float(np.linalg.eigvalsh(R0).min())]
    lam += [float(np.linalg.eigvalsh(R).min()) for (t, R, _) in trace if t < T]
    cond = [float(np.linalg.cond(Q)) for (_, _, Q) in trace]
    return lam, cond


# --------------------------------------------------------------------------
# the Muon step ([GRASP framework], [GNS §1.1 eq.(1)]; weight decay and the
# per-parameter update scale: [MuonBlog §5 item 4])
# --------------------------------------------------------------------------
def muon_step(W, M_prev, G, mu, lr, weight_decay=0.0, variant="standard",
              coeffs=None, T=5, eps=EPS, restarts=(2,), state_dtype="bf16",
              w_dtype="f32", update_scale=1.0):
    """One Muon step for a 2-D weight.  Returns (W_new, M_new, O).

    M = mu M_prev + G, rounded to ``state_dtype``; O = NS(M) (standard or
    Gram); W_new = W - lr (update_scale O + weight_decay W), rounded to
    ``w_dtype``.  The pages name the update scale without a formula, so it is
    a plain factor on O.  All arithmetic is float64 on the exact stored input
    values.  ``mu``, ``lr``, ``weight_decay`` and ``update_scale`` are used as
    given (pass the float32 values a caller hands the library to compare bit
    for bit)."""
    W = np.asarray(W, dtype=np.float64)
    M_prev = np.asarray(M_prev, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    if not (W.shape == M_prev.shape == G.shape) or W.ndim != 2:
        raise ValueError("W, M and G must be 2-D and of one shape")
    M_new = round_to(mu * M_prev + G, state_dtype)
    if variant == "standard":
        O = newton_schulz(M_new, coeffs, T, eps)
    elif variant == "gram":
        O = gram_newton_schulz(M_new, coeffs, T, eps, restarts)
    else:
        raise ValueError(f"unknown variant {variant!r}")
    W_new = round_to(W - lr * (update_scale * O + weight_decay * W), w_dtype)
    return W_new, M_new, O


# --------------------------------------------------------------------------
# FLOP formulas as the pages state them (for the library's counter tests)
# --------------------------------------------------------------------------
def counted_flops(rows, cols, variant="standard", T=5, restarts=(2,)):
    """Run the oracle on a random matrix with the counter and return
    (dense, symmetric_aware, gemm_count)."""
    rng = np.random.default_rng(0)
    M = rng.standard_normal((rows, cols))
    cnt = FlopCounter()
    if variant == "standard":
        newton_schulz(M, None, T, counter=cnt)
    else:
        gram_newton_schulz(M, None, T, restarts=restarts, counter=cnt)
    return cnt.dense, cnt.symmetric, cnt.gemms


def relative_frobenius(x, ref):
    """||x - ref||_F / ||ref||_F (the tolerance metric)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


__all__ = [
    "QUINTIC", "EPS", "round_bf16", "round_to", "FlopCounter", "newton_schulz",
    "gram_newton_schulz", "restart_diagnostics", "muon_step", "counted_flops", "relative_frobenius",
]

if __name__ == "__main__":  # pragma: no cover - manual check
    rng = np.random.default_rng(1)
    M = rng.standard_normal((256, 512))
    O1 = newton_schulz(M)
    O2 = gram_newton_schulz(M)
    print("std vs gram relF", relative_frobenius(O2, O1), math.sqrt(2))
