"""Parity for the largest launch shapes: the last product in 256-wide tiles
(n above 4096) and the last product's k-split tail (n_pad >= 8192 with a
partial last round of tiles).

* 4352 x 4600 and its transpose: n_pad = 4352 > 4096, so the last product
  (Q X or B X, which also updates W) runs in 256 x 256 tiles with the fused
  W update and O store, on inner blocks (fast form) and on the ragged last
  column block (general form); compared with the fp64 oracle in full.
* n = 8192, m = 8400 (and the transpose): the last product has 32 x 33 =
  1056 tiles on 256 compute units, so its last round of 32 tiles is cut
  along k into 8 pieces whose partials the last piece adds before the fused
  update.  The oracle's iteration at this size is ~1e13 fp64 FLOPs, so the
  input is a dyadic matrix whose singular value decomposition is known
  exactly: D[r][c] = g[r XOR c] is (H/sqrt n) diag(H g) (H/sqrt n) with H the
  Sylvester-Hadamard matrix, so Newton-Schulz maps it, by Prop. 1 of the Gram
  Newton-Schulz notes (section 2.2: the iteration acts on the singular
  values through the composed odd polynomial), to F[r][c] = f[r XOR c] with
  f = H p_5(H g / (||M||_F + eps)) / n.  The construction places D in n of
  the m columns with signs (an orthogonal change of basis on the right), and
  the closed form is pinned on the CPU against the oracle itself at n = 64.
"""
import numpy as np
import pytest
import torch

import matrix_orthogonalizing_optimizer_step_amd as mu
from oracle import muon_oracle as orc
from synth import inputs as syn

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f16": 2e-2}


def fwht(v):
    """H v for the Sylvester-Hadamard matrix, H[i][j] = (-1)^popcount(i & j),
    by the butterfly recursion H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    v = np.array(v, dtype=np.float64)
    n, h = v.shape[0], 1
    while h < n:
        a = v.reshape(-1, 2, h)
        v = np.stack([a[:, 0] + a[:, 1], a[:, 0] - a[:, 1]], axis=1).reshape(n)
        h *= 2
    return v


def dyadic_closed_form(g, src, signs, coeffs=None, T=5, eps=orc.EPS):
    """The Newton-Schulz output of syn.dyadic_matrix (n x m orientation)."""
    table = coeffs if coeffs is not None else [orc.QUINTIC] * T
    n, m = g.shape[0], src.shape[0]
    x = fwht(g) / (np.sqrt(n) * np.linalg.norm(g) + eps)
    for (a, b, c) in table:
        x = a * x + b * x ** 3 + c * x ** 5
    f = fwht(x) / n
    idx = np.arange(n, dtype=np.int32)
    F = f[np.bitwise_xor.outer(idx, idx)]
    O = np.zeros((n, m))
    cols = np.nonzero(src >= 0)[0]
    O[:, cols] = F[:, src[cols]] * signs[cols][None, :]
    return O


# ------------------------------------------------------------------ CPU pins of the closed form
@pytest.mark.parametrize("n,m", [(64, 80), (32, 32), (16, 40)])
def test_dyadic_closed_form_matches_the_oracle(n, m):
    """The closed form above equals the oracle's standard and Gram iteration
    (exact arithmetic up to fp64 rounding), in both orientations; with the
    XOR index or the Hadamard transform wrong it would not."""
    M, g, src, signs = syn.dyadic_matrix(1, n, m)
    Mf = syn.to_f64(M)
    ref = dyadic_closed_form(g, src, signs)
    assert orc.relative_frobenius(orc.newton_schulz(Mf), ref) < 1e-12
    assert orc.relative_frobenius(orc.gram_newton_schulz(Mf), ref) < 1e-12
    assert orc.relative_frobenius(orc.newton_schulz(Mf.T), ref.T) < 1e-12
    # the singular values of D are |H g|: the matrix is the stated product
    H = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(n)] for i in range(n)])
    D = g[np.bitwise_xor.outer(np.arange(n), np.arange(n))]
    assert np.allclose(H @ np.diag(H @ g) @ H / n, D, atol=1e-12)
    assert np.allclose(np.sort(np.linalg.svd(Mf, compute_uv=False)), np.sort(np.abs(fwht(g))), atol=1e-10)


# ------------------------------------------------------------------ GPU
def step_with_output(W0, G0, variant, compute):
    W = [W0.to(DEV)]
    M = [torch.zeros(G0.shape, dtype=torch.bfloat16, device=DEV)]
    O = [torch.empty(G0.shape, dtype=torch.float32, device=DEV)]  # the fp32 O the update uses
    mu.muon_step(W, M, [G0.to(DEV)], 0.95, 0.02, 0.0, variant, mu.NSConfig(compute=compute), O_out=O)
    torch.cuda.synchronize()
    return W[0].cpu(), M[0].cpu(), O[0].cpu()


def check_update(W0, W1, O1):
    """W <- W - lr O from the fp32 O, in fp32 arithmetic, rounded once to the
    weight dtype.  The kernel may contract the multiply and subtract into one
    fused operation, so the fp32 value may differ in its last bit, which can
    move a bf16 rounding by one step: bf16 weights are allowed one bf16 unit
    in the last place of the reference."""
    lr = torch.tensor(np.float32(0.02))
    ref32 = W0.float() - lr * O1
    if W0.dtype == torch.float32:
        torch.testing.assert_close(W1, ref32, rtol=2e-7, atol=2e-7)
    else:
        ulp = torch.ldexp(torch.ones_like(ref32), torch.frexp(ref32).exponent - 8)  # bf16 step at |ref|
        assert bool(((W1.float() - ref32).abs() <= ulp).all())


@pytest.mark.gpu
@pytest.mark.parametrize("shape,w_dtype,variant,compute", [
    ((4352, 4600), torch.float32, "standard", "bf16"),
    ((4600, 4352), torch.bfloat16, "standard", "bf16"),
    ((4352, 4600), torch.bfloat16, "gram", "f16"),
    ((4600, 4352), torch.float32, "gram", "f16"),
], ids=["4352x4600-std-f32W", "4600x4352-std-bf16W", "4352x4600-gram-bf16W", "4600x4352-gram-f32W"])
def test_wide_last_product_against_oracle(shape, w_dtype, variant, compute):
    r, c = shape
    print(f"wide last product {shape} {variant}/{compute} W {w_dtype}", flush=True)
    W0 = syn.random_matrix(90, r, c, dtype="bf16" if w_dtype == torch.bfloat16 else "f32")
    G0 = syn.random_matrix(91, r, c, std=1e-3, dtype="bf16")
    W1, M1, O1 = step_with_output(W0, G0, variant, compute)
    assert torch.equal(M1, G0)  # M_prev = 0: the stored momentum is G
    Mf = syn.to_f64(G0)
    ref = orc.newton_schulz(Mf) if variant == "standard" else orc.gram_newton_schulz(Mf)
    err = orc.relative_frobenius(syn.to_f64(O1), ref)
    print(f"  relF {err:.3e}", flush=True)
    assert err < TOL[compute]
    check_update(W0, W1, O1)


@pytest.mark.gpu
@pytest.mark.parametrize("transposed", [False, True], ids=["8192x8400", "8400x8192"])
@pytest.mark.parametrize("variant,compute", [("standard", "bf16"), ("gram", "f16")])
def test_last_product_tail_split_against_closed_form(transposed, variant, compute):
    n, m = 8192, 8400
    print(f"tail-split last product n={n} m={m} transposed={transposed} {variant}/{compute}", flush=True)
    G0, g, src, signs = syn.dyadic_matrix(3, n, m)
    ref = dyadic_closed_form(g, src, signs)
    if transposed:
        G0, ref = G0.T.contiguous(), ref.T
    W0 = syn.random_matrix(92, *G0.shape)
    W1, M1, O1 = step_with_output(W0, G0, variant, compute)
    assert torch.equal(M1, G0)
    err = orc.relative_frobenius(syn.to_f64(O1), ref)
    print(f"  relF {err:.3e}", flush=True)
    assert err < TOL[compute]
    check_update(W0, W1, O1)
