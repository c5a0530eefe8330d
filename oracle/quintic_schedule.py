"""Oracle for per-iteration quintic schedules (test infrastructure only).

Only the test suite may import this module; the library never does, and it
shares no code with the library's own derivation (a Remez exchange in C++).

Sources:

* [GNS §3.2] ("优化器 (3)（Gram Newton-Schulz）", restarts): Gram
  Newton-Schulz is run with the Polar Express quintics, one odd polynomial
  p_t(x) = a_t x + b_t x^3 + c_t x^5 per iteration.  The printed table is
  garbled (p_1(1) = 2.27, and the printed schedule diverges), so the schedule
  is rebuilt from the method's principle: p_t is the odd quintic nearest to
  the constant 1 in the maximum norm on the interval [l_t, u_t] that holds the
  singular values before iteration t, starting from [ell, 1], and the next
  interval is the image of the current one under the applied polynomial.
* [GNS §3.3] (further safety measures): a safety factor that keeps the
  iteration convergent for singular values up to 1.05.  Its equation is lost;
  the reading is p_t(x) -> p_t(x / f), i.e. (a / f, b / f^3, c / f^5).

Readings (also in the design notes): the minimax problem is solved as a
linear programme on a dense grid (the plain definition: minimise the largest
error); once the interval is narrower than 1e-2 relative, the polynomial is
the limit (15/8, -10/8, 3/8) fixed by p(1) = 1, p'(1) = p''(1) = 0 (its
error there is below 3e-6, under any 16-bit rounding); the
coefficients are rounded to fp32 and the intervals follow the rounded
polynomials.
"""
from __future__ import annotations

import numpy as np
from scipy.optimize import linprog

LIMIT = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)
NARROW = 1e-2


def quintic(coeffs, x):
    a, b, c = coeffs
    x = np.asarray(x, dtype=np.float64)
    return a * x + b * x ** 3 + c * x ** 5


def _grid(s, n=20001):
    """Points of [s, 1]: uniform plus geometric (dense near a small s)."""
    g = np.concatenate([np.linspace(s, 1.0, n), np.geomspace(s, 1.0, n // 4)])
    return np.unique(g)


def minimax_quintic(l, u, n=20001):
    """The odd quintic minimising max |1 - p(x)| over x in [l, u] (0 < l < u),
    as a linear programme over a dense grid of [l / u, 1], then scaled back
    to [l, u].
    Returns ((a, b, c), E)."""
    s = l / u
    x = _grid(s, n)
    # p(x) = x q(x^2) with q written in the centred variable w = (x^2 - m) / h
    # that spans [-1, 1] on the interval (a well-conditioned basis even for
    # narrow intervals); expanded back to monomials at the end
    m, h = (1.0 + s * s) / 2.0, (1.0 - s * s) / 2.0
    w = (x * x - m) / h
    V = np.stack([x, x * w, x * w * w], axis=1)
    ones = np.ones((len(x), 1))
    # variables (alpha, beta, gamma, E); minimise E subject to -E <= 1 - p <= E
    A_ub = np.vstack([np.hstack([-V, -ones]), np.hstack([V, -ones])])
    b_ub = np.concatenate([-np.ones(len(x)), np.ones(len(x))])
    res = linprog(np.array([0.0, 0.0, 0.0, 1.0]), A_ub=A_ub, b_ub=b_ub,
                  bounds=[(None, None)] * 3 + [(0.0, None)], method="highs",
                  options={"primal_feasibility_tolerance": 1e-10, "dual_feasibility_tolerance": 1e-10})
    if not res.success:
        raise RuntimeError(f"minimax LP failed on [{l}, {u}]: {res.message}")
    al, be, ga, E = res.x
    # q(y) = al + be (y - m) / h + ga ((y - m) / h)^2 = c0 + c1 y + c2 y^2
    c2 = ga / (h * h)
    c1 = be / h - 2.0 * ga * m / (h * h)
    c0 = al - be * m / h + ga * m * m / (h * h)
    return (c0 / u, c1 / u ** 3, c2 / u ** 5), float(E)


def image(coeffs, l, u):
    """[min p, max p] over [l, u]: the ends and the critical points inside."""
    a, b, c = coeffs
    pts = [l, u]
    # p'(x) = a + 3 b x^2 + 5 c x^4, a quadratic in x^2
    for y in np.roots([5.0 * c, 3.0 * b, a]):
        if abs(y.imag) < 1e-12 and y.real > 0:
            x = np.sqrt(y.real)
            if l < x < u:
                pts.append(x)
    v = quintic(coeffs, np.array(pts))
    return float(v.min()), float(v.max())


def schedule(T, ell=1e-3, safety=1.0):
    """T applied polynomials (fp32 values) and the T + 1 intervals."""
    l, u = float(ell), 1.0
    coeffs, bounds = [], [(l, u)]
    for _ in range(T):
        if (u - l) <= NARROW * u:
            p = LIMIT
        else:
            p, _ = minimax_quintic(l, u)
        f = float(safety)
        p = tuple(float(np.float32(v)) for v in (p[0] / f, p[1] / f ** 3, p[2] / f ** 5))
        coeffs.append(p)
        l, u = image(p, l, u)
        bounds.append((l, u))
    return coeffs, bounds
