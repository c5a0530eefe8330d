"""Pins for the fp64 oracle: closed forms, invariants, exact counts and
special cases fixed by the Gram Newton-Schulz notes and by linear algebra.
None of these re-types the oracle's own formula; each would fail for a
dropped term, a wrong sign, a transposed operand or a wrong loop range."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import muon_oracle as orc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
ABC = tuple(GOLDEN["quintic_coefficients"]["value"])


def scalar_map(x, coeffs):
    """Prop.1 of the Gram NS notes: on singular values the iteration is the
    composition of the odd polynomials p_t(x) = a x + b x^3 + c x^5."""
    x = np.asarray(x, dtype=np.float64)
    for (a, b, c) in coeffs:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def closed_form(M, coeffs, eps=1e-7):
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    x = s / (np.linalg.norm(M) + eps)
    return (U * scalar_map(x, coeffs)[None, :]) @ Vt


def rng(seed):
    return np.random.default_rng(1234 + seed)


# ---------------------------------------------------------------- constants
def test_constants_match_pages():
    assert orc.QUINTIC == ABC
    assert orc.EPS == GOLDEN["eps"]["value"]


# ---------------------------------------------------------------- rounding
def test_bf16_rounding_ties_and_single_rounding():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: one,                      # tie -> even (1.0)
        one + 1.5 * ulp: one + 2 * ulp,          # tie -> even mantissa
        one + ulp / 2 + 2.0 ** -40: one + ulp,   # just above the tie: one rounding only
        -(one + ulp / 2 + 2.0 ** -40): -(one + ulp),
        3.0e38 * 2: np.inf,
        0.0: 0.0,
    }
    got = orc.round_bf16(np.array(list(cases.keys())))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))


def test_bf16_rounding_matches_torch_on_float32_values():
    # values that are exact in fp32: torch's fp32->bf16 conversion is RNE
    x = rng(0).standard_normal(100000).astype(np.float32) * np.float32(1e-3)
    x[:100] = np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(100, dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_bf16(x.astype(np.float64)), ref)


def test_bf16_rounding_of_non_contiguous_input():
    # a transposed view and a strided slice give the rounding of their own
    # elements in their own positions (an element-order slip would scramble them)
    one, ulp = 1.0, 2.0 ** -7
    A = np.array([[one + ulp / 2, 3.0, -(one + 1.5 * ulp)],
                  [0.0, one + ulp / 2 + 2.0 ** -40, 5.0e-39]])
    want = np.array([[one, 3.0, -(one + 2 * ulp)],
                     [0.0, one + ulp, np.round(5.0e-39 / 2.0 ** -133) * 2.0 ** -133]])
    np.testing.assert_array_equal(orc.round_bf16(A.T), want.T)
    np.testing.assert_array_equal(orc.round_bf16(A[:, ::2]), want[:, ::2])
    x = rng(7).standard_normal((37, 53)).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(np.ascontiguousarray(x.T)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_bf16(x.T), ref)
    np.testing.assert_array_equal(orc.round_bf16(x[::3, 1::2]), orc.round_bf16(x)[::3, 1::2])


def test_relative_frobenius_hand_values():
    # ||x - ref||_F / ||ref||_F with values worked out by hand; pairs of equal
    # norm and nonzero difference rule out a comparison of norms alone
    I4 = np.eye(4)
    assert orc.relative_frobenius(-I4, I4) == pytest.approx(2.0, abs=1e-15)
    assert orc.relative_frobenius(I4, I4) == 0.0
    E = np.array([[0.0, 1.0, 0.0, 0.0], [0.0, 0.0, 0.0, 2.0], [0.0, 0.0, 0.0, 0.0], [2.0, 0.0, 0.0, 0.0]])
    assert orc.relative_frobenius(I4 + E, I4) == pytest.approx(3.0 / 2.0, abs=1e-15)  # ||E|| = 3, ||I4|| = 2
    # a permutation of the entries: same norm, distance sqrt(2) of the norm
    a, b = np.array([[1.0, 0.0], [0.0, 0.0]]), np.array([[0.0, 1.0], [0.0, 0.0]])
    assert orc.relative_frobenius(a, b) == pytest.approx(np.sqrt(2.0), abs=1e-15)
    # the reference is the second argument: the metric is not symmetric
    assert orc.relative_frobenius(np.array([[3.0]]), np.array([[1.0]])) == pytest.approx(2.0)
    assert orc.relative_frobenius(np.array([[1.0]]), np.array([[3.0]])) == pytest.approx(2.0 / 3.0)
    # a rotation by 90 degrees of a 2-vector: |x| = |ref| = 5, |x - ref| = 5 sqrt(2)
    assert orc.relative_frobenius(np.array([[-4.0, 3.0]]), np.array([[3.0, 4.0]])) == pytest.approx(np.sqrt(2.0))
    # an all-zero reference: the plain norm of the difference
    assert orc.relative_frobenius(np.array([[3.0, 4.0]]), np.zeros((1, 2))) == pytest.approx(5.0)
    # transposed inputs compare position by position
    x = np.array([[1.0, 2.0, 0.0]])
    assert orc.relative_frobenius(x.T, x.T.copy()) == 0.0
    assert orc.relative_frobenius(x[:, ::-1], x) == pytest.approx(np.sqrt(2.0 / 5.0))  # [0, 2, 1] - [1, 2, 0]


def test_round_to_idempotent_and_dtypes():
    x = rng(1).standard_normal(1000)
    for dt in ("f32", "bf16", "f16"):
        y = orc.round_to(x, dt)
        np.testing.assert_array_equal(orc.round_to(y, dt), y)
    assert np.array_equal(orc.round_to(x, "f64"), x)


# ---------------------------------------------------------------- Prop.1 closed form
@pytest.mark.parametrize("shape", [(8, 8), (5, 13), (13, 5), (32, 96), (96, 32), (64, 64), (1, 17)])
def test_standard_ns_matches_singular_value_closed_form(shape):
    M = rng(2).standard_normal(shape)
    O = orc.newton_schulz(M)
    ref = closed_form(M, [ABC] * 5)
    assert orc.relative_frobenius(O, ref) < 1e-12


def test_closed_form_holds_for_any_coefficient_table():
    M = rng(3).standard_normal((24, 40))
    table = [(2.0, -1.5, 0.5), (3.0, -3.2, 1.2), (1.5, -0.5, 0.0), (2.5, -2.0, 0.6)]
    O = orc.newton_schulz(M, coeffs=table, T=4)
    assert orc.relative_frobenius(O, closed_form(M, table)) < 1e-12


def test_coefficient_order_matters():
    # a transposed (a, b, c) would break the closed form
    M = rng(4).standard_normal((16, 24))
    bad = closed_form(M, [(ABC[2], ABC[1], ABC[0])] * 5)
    assert orc.relative_frobenius(orc.newton_schulz(M), bad) > 1e-2


# ---------------------------------------------------------------- textbook polar
@pytest.mark.parametrize("shape", [(2, 3), (6, 6), (7, 19), (16, 40), (40, 16)])
def test_convergent_polynomial_reaches_exact_polar(shape):
    """With h(y) = 15/8 - 10/8 y + 3/8 y^2 (Prop.2 proof) the iteration
    converges to U V^T, the polar factor of Definition 1."""
    r, c = shape
    k = min(r, c)
    U, _ = np.linalg.qr(rng(5).standard_normal((r, k)))
    V, _ = np.linalg.qr(rng(6).standard_normal((c, k)))
    s = np.linspace(1.0, 0.05, k)  # well conditioned: sigma_min / ||M|| >= 1e-2
    M = (U * s) @ V.T
    h = tuple(GOLDEN["cubic_ns_h"]["value"])
    O = orc.newton_schulz(M, coeffs=[h] * 30, T=30)
    Uf, _, Vtf = np.linalg.svd(M, full_matrices=False)
    assert orc.relative_frobenius(O, Uf @ Vtf) < 1e-12
    Og = orc.gram_newton_schulz(M, coeffs=[h] * 30, T=30, restarts=(5, 10, 15, 20, 25))
    assert orc.relative_frobenius(Og, Uf @ Vtf) < 1e-12


# ---------------------------------------------------------------- Gram == standard
@pytest.mark.parametrize("restarts", [(), (2,), (1, 2, 3, 4), (3,), (1,)])
@pytest.mark.parametrize("shape", [(12, 30), (30, 12), (20, 20)])
def test_gram_equals_standard_in_exact_arithmetic(restarts, shape):
    M = rng(7).standard_normal(shape)
    O1 = orc.newton_schulz(M)
    O2 = orc.gram_newton_schulz(M, restarts=restarts)
    assert orc.relative_frobenius(O2, O1) < 1e-12


def test_gram_equals_standard_other_tables_and_T():
    M = rng(8).standard_normal((10, 26))
    table = [(2.0, -1.5, 0.5), (3.0, -3.2, 1.2), (1.5, -0.5, 0.0), (2.5, -2.0, 0.6), (1.9, -1.1, 0.2), (1.2, -0.3, 0.1)]
    for restarts in [(), (2,), (3, 4)]:
        assert orc.relative_frobenius(orc.gram_newton_schulz(M, table, T=6, restarts=restarts),
                                      orc.newton_schulz(M, table, T=6)) < 1e-12


# ---------------------------------------------------------------- Thm.1 scalar form
def test_gram_diagonal_input_follows_scalar_recursion():
    """For a diagonal X0 every Gram state is diagonal: R_t = diag(x_t^2) and
    Q_T = diag(x_T / x_0) (Theorem 1)."""
    d = np.array([0.9, 0.5, 0.2, 0.05, 0.01, 0.3])
    M = np.diag(d)
    trace = []
    orc.gram_newton_schulz(M, restarts=(), trace=trace)
    x0 = d / (np.linalg.norm(d) + 1e-7)
    xs = [x0]
    for t in range(5):
        xs.append(scalar_map(xs[-1], [ABC]))
    for (t, R, Q) in trace:
        if t < 5:
            np.testing.assert_allclose(R, np.diag(xs[t] ** 2), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(Q, np.diag(xs[t] / x0), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- Prop.2 spurious negative eigenvalue
@pytest.mark.parametrize("h", [ABC, (1.875, -1.25, 0.375)])
def test_negative_eigenvalue_grows_geometrically(h):
    lam = GOLDEN["spurious_eigenvalue_bf16"]["value"]
    R0 = np.diag([lam, 0.3, 0.2, 0.1])
    trace = []
    orc.gram_newton_schulz(np.eye(4), coeffs=[h] * 5, restarts=(), R0=R0, trace=trace)
    r = lam
    mags = []
    for (t, R, _) in trace[:-1]:
        a, b, c = h
        r = r * (a + b * r + c * r * r) ** 2
        assert R[0, 0] == pytest.approx(r, rel=1e-9)
        assert R[0, 0] < 0
        mags.append(abs(R[0, 0]))
    ratios = np.array(mags[1:]) / np.array(mags[:-1])
    assert np.all(ratios > (h[0] ** 2) * 0.99)  # at least a^2 per step
    # the spurious entry does not leak into the other eigenvalues
    assert abs(trace[-2][1][0, 1]) == 0.0


def test_restart_removes_negative_eigenvalue():
    M = rng(9).standard_normal((6, 10))
    R0 = M @ M.T / (np.linalg.norm(M) + 1e-7) ** 2
    w, V = np.linalg.eigh(R0)
    w[0] = -1e-5
    R0 = (V * w) @ V.T
    trace = []
    orc.gram_newton_schulz(M, restarts=(2,), R0=R0, trace=trace)
    R_after = trace[1][1]  # R right after the restart is X X^T
    assert np.linalg.eigvalsh(R_after).min() > -1e-12


# ---------------------------------------------------------------- FLOP counts
def _n3(n):
    return n ** 3


@pytest.mark.parametrize("n,alpha", [(8, 1), (8, 2), (8, 4), (4, 8), (6, 3)])
def test_flop_counts_match_pages(n, alpha):
    m = alpha * n
    g = GOLDEN
    d, s, k = orc.counted_flops(n, m, "standard")
    assert d == (g["standard_ns_T5"]["dense_coeff_alpha"] * alpha + g["standard_ns_T5"]["dense_coeff_const"]) * _n3(n)
    assert k == g["standard_ns_T5"]["gemms"]
    assert s == 5 * (g["standard_ns_symmetric"]["per_iteration_alpha"] * alpha + g["standard_ns_symmetric"]["per_iteration_const"]) * _n3(n)
    _, s, k = orc.counted_flops(n, m, "gram", restarts=())
    assert s == (g["naive_gram_T5"]["coeff_const"] + g["naive_gram_T5"]["coeff_alpha"] * alpha) * _n3(n)
    assert k == g["naive_gram_T5"]["gemms"]
    _, s1, k1 = orc.counted_flops(n, m, "gram", restarts=(2,))
    extra = (g["restart_extra_products"]["QX"] + g["restart_extra_products"]["XXt"]) * alpha * _n3(n)
    saved = (g["restart_saved_products"]["R2"] + g["restart_saved_products"]["Q3"]) * _n3(n)
    assert s1 == s + extra - saved
    assert k1 == k + 2 - 3
    # transposed orientation counts the same
    assert orc.counted_flops(m, n, "gram", restarts=(2,))[1] == s1
    # a restart can only follow an iteration t < T: asking for t = T changes nothing
    assert orc.counted_flops(n, m, "gram", restarts=(5,))[1:] == (s, k)


def test_savings_percentages_match_pages():
    g = GOLDEN
    n, alpha = 8, 4
    _, sym_std, _ = orc.counted_flops(n, alpha * n, "standard")
    dense_std, _, _ = orc.counted_flops(n, alpha * n, "standard")
    _, naive, _ = orc.counted_flops(n, alpha * n, "gram", restarts=())
    _, rest, _ = orc.counted_flops(n, alpha * n, "gram", restarts=(2,))
    pct = lambda new, old: round(100 * (1 - new / old))
    assert pct(naive, sym_std) == g["naive_gram_alpha4_savings_pct"]["vs_symmetric_standard"]
    assert pct(naive, dense_std) == g["naive_gram_alpha4_savings_pct"]["vs_typical"]
    assert pct(rest, sym_std) == g["restart_gram_alpha4_savings_pct"]["vs_symmetric_standard"]
    assert pct(rest, dense_std) == g["restart_gram_alpha4_savings_pct"]["vs_typical"]
    assert pct(rest, sym_std) == g["alpha4_savings_pct_5_2"]["value"]
    _, sym1, _ = orc.counted_flops(n, n, "standard")
    _, rest1, _ = orc.counted_flops(n, n, "gram", restarts=(2,))
    assert pct(rest1, sym1) == g["square_savings_pct"]["value"]


# ---------------------------------------------------------------- special cases
def test_zero_matrix_gives_zero():
    for f in (orc.newton_schulz, orc.gram_newton_schulz):
        O = f(np.zeros((5, 9)))
        assert np.all(O == 0) and np.all(np.isfinite(O))


def test_rank_one():
    u = rng(10).standard_normal(7)
    v = rng(11).standard_normal(15)
    M = 3.0 * np.outer(u, v)
    x = np.linalg.norm(M) / (np.linalg.norm(M) + 1e-7)
    ref = scalar_map(x, [ABC] * 5) * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    for f in (orc.newton_schulz, orc.gram_newton_schulz):
        assert orc.relative_frobenius(f(M), ref) < 1e-12
    assert scalar_map(1.0, [ABC] * 5) == pytest.approx(0.696436, abs=1e-6)


@pytest.mark.parametrize("n", [4, 16, 64])
def test_scaled_orthogonal(n):
    Qm, _ = np.linalg.qr(rng(12).standard_normal((n, n)))
    M = 2.5 * Qm
    x = 2.5 / (2.5 * np.sqrt(n) + 1e-7)
    ref = scalar_map(x, [ABC] * 5) * Qm
    for f in (orc.newton_schulz, orc.gram_newton_schulz):
        assert orc.relative_frobenius(f(M), ref) < 1e-12


def test_row_vector():
    v = rng(13).standard_normal((1, 23))
    ref = scalar_map(1.0 - 1e-7 / (np.linalg.norm(v) + 1e-7), [ABC] * 5) * v / np.linalg.norm(v)
    assert orc.relative_frobenius(orc.newton_schulz(v), ref) < 1e-12
    assert orc.relative_frobenius(orc.newton_schulz(v.T), ref.T) < 1e-12


def test_orientation_invariance():
    M = rng(14).standard_normal((18, 44))
    assert orc.relative_frobenius(orc.newton_schulz(M.T), orc.newton_schulz(M).T) < 1e-12
    assert orc.relative_frobenius(orc.gram_newton_schulz(M.T), orc.gram_newton_schulz(M).T) < 1e-12


def test_singular_values_in_band():
    # sup of p_5 on [0, 1] and the band for x >= 0.0015 (independent grid search)
    grid = np.linspace(0.0, 1.0, 2_000_001)
    p = scalar_map(grid, [ABC] * 5)
    sup = p.max()
    lo = p[grid >= 0.0015051].min()
    assert sup == pytest.approx(1.202369, abs=2e-6)
    assert lo == pytest.approx(0.681831, abs=2e-6)
    M = rng(15).standard_normal((64, 256))
    sv = np.linalg.svd(orc.newton_schulz(M), compute_uv=False)
    x = np.linalg.svd(M, compute_uv=False) / np.linalg.norm(M)
    assert x.min() > 0.0015051
    assert sv.min() >= lo - 1e-12 and sv.max() <= sup + 1e-12


# ---------------------------------------------------------------- the Muon step
def test_muon_step_momentum_and_update():
    r = rng(16)
    W = r.standard_normal((12, 20))
    Mp = orc.round_bf16(r.standard_normal((12, 20)))
    G = orc.round_bf16(r.standard_normal((12, 20)) * 1e-3)
    mu, lr, wd = float(np.float32(0.95)), float(np.float32(0.02)), 0.1
    W1, M1, O = orc.muon_step(W, Mp, G, mu, lr, wd, state_dtype="bf16", w_dtype="f64")
    # the momentum is stored in bf16 and is within half an ulp of the exact value
    exact = mu * Mp + G
    assert np.array_equal(orc.round_bf16(M1), M1)
    spacing = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert np.all(np.abs(M1 - exact) <= spacing / 2 + 1e-300)
    # O is the orthogonalisation of the stored momentum
    assert orc.relative_frobenius(O, closed_form(M1, [ABC] * 5)) < 1e-12
    # the update direction is -lr (O + wd W)
    np.testing.assert_allclose(W1, W - lr * O - lr * wd * W, rtol=0, atol=1e-14)


def test_muon_step_first_step_and_zero_gradient():
    r = rng(17)
    W = orc.round_to(r.standard_normal((6, 6)), "f32")
    G = orc.round_bf16(r.standard_normal((6, 6)))
    W1, M1, _ = orc.muon_step(W, np.zeros((6, 6)), G, 0.95, 0.02, state_dtype="bf16")
    assert np.array_equal(M1, G)  # M_0 = 0, first momentum is the gradient
    W2, M2, O2 = orc.muon_step(W, np.zeros((6, 6)), np.zeros((6, 6)), 0.95, 0.02)
    assert np.all(O2 == 0) and np.array_equal(W2, W)


def test_muon_step_identity_momentum():
    n = 16
    W = np.zeros((n, n))
    G = np.eye(n)
    W1, _, _ = orc.muon_step(W, np.zeros((n, n)), G, 0.9, 0.5, state_dtype="f32", w_dtype="f64")
    x = 1.0 / (np.sqrt(n) + 1e-7)
    np.testing.assert_allclose(W1, -0.5 * scalar_map(x, [ABC] * 5) * np.eye(n), atol=1e-14)


def test_muon_step_update_scale_closed_forms():
    # [MuonBlog §5 item 4]: W <- W - lr (s O + wd W).  s = 0 leaves pure
    # decoupled decay W (1 - lr wd) although O != 0; with W = 0 and identity
    # momentum the update is -lr s p_5(x) I (the scalar map of the quintic).
    r = rng(19)
    W = r.standard_normal((8, 24))
    G = r.standard_normal((8, 24))
    W1, _, O = orc.muon_step(W, np.zeros_like(W), G, 0.95, 0.02, 0.1, state_dtype="f64", w_dtype="f64",
                             update_scale=0.0)
    assert np.abs(O).max() > 0.1
    np.testing.assert_allclose(W1, W * (1.0 - 0.02 * 0.1), rtol=0, atol=1e-15)
    n = 16
    for s in (0.5, 2.5):
        W1, _, _ = orc.muon_step(np.zeros((n, n)), np.zeros((n, n)), np.eye(n), 0.9, 0.5, state_dtype="f32",
                                 w_dtype="f64", update_scale=s)
        x = 1.0 / (np.sqrt(n) + 1e-7)
        np.testing.assert_allclose(W1, -0.5 * s * scalar_map(x, [ABC] * 5) * np.eye(n), atol=1e-14)


def test_muon_step_gram_variant_equals_standard():
    r = rng(18)
    W = r.standard_normal((10, 30))
    G = r.standard_normal((10, 30))
    a = orc.muon_step(W, np.zeros_like(W), G, 0.95, 0.02, variant="standard", state_dtype="f64", w_dtype="f64")
    b = orc.muon_step(W, np.zeros_like(W), G, 0.95, 0.02, variant="gram", state_dtype="f64", w_dtype="f64")
    assert orc.relative_frobenius(b[2], a[2]) < 1e-12


def test_rejects_non_2d():
    with pytest.raises(ValueError):
        orc.newton_schulz(np.zeros(5))
    with pytest.raises(ValueError):
        orc.muon_step(np.zeros((2, 2)), np.zeros((2, 3)), np.zeros((2, 2)), 0.9, 0.1)
