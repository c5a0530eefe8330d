"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances are the relative Frobenius errors the design fixes: 2e-2 for
16-bit MFMA operands and 1e-4 for the fp32 check path (fp32 operands, fp64
accumulation).  Momentum updates must match bit for bit."""
import numpy as np
import pytest
import torch

import matrix_orthogonalizing_optimizer_step_amd as mu
from oracle import muon_oracle as orc
from synth import inputs as syn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}
QUINTIC5 = [orc.QUINTIC] * 5


def mask_of(restarts):
    return sum(1 << (t - 1) for t in restarts)


def gpu_orth(variant, Ms, compute, T=5, coeffs=None, restarts=(2,), shift=True, odt=torch.float32):
    cfg = mu.NSConfig(T=T, coeffs=coeffs, compute=compute, shift=shift,
                      restart_mask=mask_of(restarts) if variant == "gram" else None)
    M = [m.to(DEV) for m in Ms]
    O = [torch.empty(m.shape, dtype=odt, device=DEV) for m in Ms]
    f = mu.ns_orthogonalize if variant == "standard" else mu.gram_ns_orthogonalize
    f(M, O, cfg)
    torch.cuda.synchronize()
    return [syn.to_f64(o) for o in O]


def oracle_orth(variant, M, T=5, coeffs=None, restarts=(2,)):
    M = syn.to_f64(M)
    if variant == "standard":
        return orc.newton_schulz(M, coeffs, T)
    return orc.gram_newton_schulz(M, coeffs, T, restarts=restarts)


def relF(a, b):
    return orc.relative_frobenius(a, b)


# Precision tracking: beside the design tolerance, each parity case below
# holds a bound in units of its operand type's unit roundoff u (bf16 2^-8,
# fp16 2^-11, fp32 2^-24), so that a loss of precision well inside the design
# tolerance still fails.  Square matrices get a larger multiple (X X^T then
# has the squared condition number of X); the Gram iteration without restarts
# on a square matrix is the case the Gram NS notes warn about (section 3.2)
# and keeps the design tolerance only, as do bf16 operands on squares.
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}


def tracked_bound(variant, compute, shape, restarts=(2,)):
    square = shape[0] == shape[1] and shape[0] > 1
    if square and (compute == "bf16" or (variant == "gram" and not restarts)):
        return TOL[compute]
    if compute == "f32":
        mult = 64 if square else 16
    elif compute == "f16":
        mult = (20 if variant == "gram" else 6) if square else 6
    else:
        mult = 4
    return min(TOL[compute], mult * UNIT[compute])


# ------------------------------------------------------------------ single products
@pytest.mark.parametrize("compute", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(256, 512), (200, 300), (300, 200)])
@pytest.mark.parametrize("abc", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.7, -0.4, 0.3)])
def test_one_iteration_with_probe_coefficients(compute, shape, abc):
    """T = 1 isolates the products: (1,0,0) is the normalisation alone,
    (0,1,0) is X X^T X, (0,0,1) is (X X^T)^2 X."""
    M = syn.random_matrix(1, *shape)
    if compute == "bf16":  # bf16 operands take the fixed quintic only
        with pytest.raises(mu.MuonError) as e:
            gpu_orth("standard", [M], compute, T=1, coeffs=[abc])
        assert e.value.status == 2
        return
    for shift in (True, False):
        got = gpu_orth("standard", [M], compute, T=1, coeffs=[abc], shift=shift)[0]
        ref = oracle_orth("standard", M, T=1, coeffs=[abc])
        tol = 1e-5 if compute == "f32" else 1e-2
        assert relF(got, ref) < tol, (compute, shape, abc, shift, relF(got, ref))


# ------------------------------------------------------------------ full iterations
SHAPES = [(256, 512), (512, 256), (100, 300), (300, 100), (257, 513), (1, 64), (64, 1), (33, 33), (384, 384)]


@pytest.mark.parametrize("compute", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_standard_ns_parity(compute, shape):
    M = syn.random_matrix(2, *shape, std=1e-3, dtype="bf16")
    got = gpu_orth("standard", [M], compute)[0]
    ref = oracle_orth("standard", M)
    assert relF(got, ref) < tracked_bound("standard", compute, shape), relF(got, ref)


@pytest.mark.parametrize("compute", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("restarts", [(2,), (), (1, 2, 3, 4)])
@pytest.mark.parametrize("shape", SHAPES)
def test_gram_ns_parity(compute, restarts, shape):
    M = syn.random_matrix(3, *shape, std=1e-3, dtype="bf16")
    if compute == "bf16":  # Gram NS computes in float16; bf16 is refused (outside 2e-2 on squares)
        with pytest.raises(mu.MuonError) as e:
            gpu_orth("gram", [M], compute, restarts=restarts)
        assert e.value.status == 2
        return
    got = gpu_orth("gram", [M], compute, restarts=restarts)[0]
    ref = oracle_orth("gram", M, restarts=restarts)
    assert relF(got, ref) < tracked_bound("gram", compute, shape, restarts), relF(got, ref)


@pytest.mark.parametrize("f", [1.0, 1.05])
@pytest.mark.parametrize("variant,compute", [("standard", "f16"), ("standard", "f32"), ("gram", "f16"),
                                             ("gram", "f32")])
def test_quintic_schedule_parity(variant, compute, f):
    """Per-iteration minimax quintics from the library's schedule (ell = 1e-3,
    with and without the safety factor), restart after iteration 2 for Gram,
    against the oracle run with the same fp32 coefficients.  The steep first
    polynomials amplify operand rounding: bf16 operands measured up to 2.6e-2
    on 700 x 256, over the 16-bit tolerance, so the library refuses bf16 with
    such a table and the 16-bit case runs with the fp16 operands that the Gram
    NS notes recommend (section 3.3)."""
    coeffs, _ = mu.quintic_schedule(5, 1e-3, f)
    for shape in ((300, 1100), (700, 256)):
        M = syn.random_matrix(50, *shape, std=1e-3, dtype="bf16")
        got = gpu_orth(variant, [M], compute, coeffs=coeffs)[0]
        ref = oracle_orth(variant, M, coeffs=coeffs)
        assert relF(got, ref) < TOL[compute], shape


def test_batch_matches_single_calls_bitwise():
    Ms = [syn.random_matrix(10 + i, 200, 456, dtype="bf16") for i in range(3)]
    for variant in ("standard", "gram"):
        batched = gpu_orth(variant, Ms, None)
        for i, M in enumerate(Ms):
            single = gpu_orth(variant, [M], None)[0]
            assert np.array_equal(batched[i], single)


def test_deterministic():
    M = syn.random_matrix(20, 384, 640, dtype="bf16")
    for variant in ("standard", "gram"):
        a = gpu_orth(variant, [M], None)[0]
        b = gpu_orth(variant, [M], None)[0]
        assert np.array_equal(a, b)


@pytest.mark.parametrize("shape", [(256, 8192), (300, 9000), (9000, 300)])
def test_tail_split_long_k(shape):
    """X X^T with k >= 8192 on fewer tiles than compute units is cut along k;
    the pieces' fp32 partials are added in a fixed order: oracle parity and
    bitwise repeatability."""
    M = syn.random_matrix(22, *shape, dtype="bf16")
    for variant, compute in (("standard", "bf16"), ("gram", "f16")):
        a = gpu_orth(variant, [M], compute)[0]
        b = gpu_orth(variant, [M], compute)[0]
        assert np.array_equal(a, b)
        assert relF(a, oracle_orth(variant, M)) < TOL[compute]


@pytest.mark.parametrize("shape", [(1, 1 << 20), (1 << 20, 1)], ids=["row-2^20", "column-2^20"])
def test_maximum_dimension_vector(shape):
    """The largest dimension the ABI accepts (2^20), on the degenerate n = 1
    case: X X^T is 1 x 1 with k = 2^20 (cut into k pieces), and O is
    p_5(x) v / ||v|| with x = ||v|| / (||v|| + eps)."""
    M = syn.random_matrix(23, *shape, std=1e-3, dtype="bf16")
    v = syn.to_f64(M).reshape(-1)
    x = np.linalg.norm(v) / (np.linalg.norm(v) + orc.EPS)
    for _ in range(5):
        x = QUINTIC5[0][0] * x + QUINTIC5[0][1] * x ** 3 + QUINTIC5[0][2] * x ** 5
    closed = (x * v / np.linalg.norm(v)).reshape(shape)
    for variant, compute in (("standard", "bf16"), ("gram", "f16")):
        got = gpu_orth(variant, [M], compute)[0]
        ref = oracle_orth(variant, M)
        assert relF(ref, closed) < 1e-12
        assert relF(got, ref) < TOL[compute], (variant, relF(got, ref))


def test_zero_matrix_gives_zero():
    M = torch.zeros(64, 96, dtype=torch.bfloat16)
    for variant in ("standard", "gram"):
        O = gpu_orth(variant, [M], None)[0]
        assert np.all(O == 0)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
@pytest.mark.parametrize("variant", ["standard", "gram"])
def test_non_finite_momentum_propagates(variant, bad):
    """A NaN or Inf in the gradient propagates: the stored momentum holds it
    at its own position only (bit for bit against the oracle's rounding), and
    the norm, hence every entry of O and of the updated W, becomes NaN, as the
    fp64 oracle's IEEE arithmetic gives (Inf / ||M|| = Inf / Inf).  The
    device stays usable: a finite step right after matches the oracle."""
    r, c = 300, 520
    W = syn.random_matrix(95, r, c)
    G = syn.random_matrix(96, r, c, std=1e-3, dtype="bf16")
    G[17, 401] = bad
    Mp = torch.zeros(r, c, dtype=torch.bfloat16)
    W1, M1, O1 = run_step([W], [Mp], [G], 0.95, 0.02, 0.0, variant)
    Wr, Mr, Or = orc.muon_step(syn.to_f64(W), syn.to_f64(Mp), syn.to_f64(G), float(np.float32(0.95)),
                               float(np.float32(0.02)), 0.0, variant, state_dtype="bf16", w_dtype="f64")
    assert np.array_equal(syn.to_f64(M1[0]), Mr, equal_nan=True)
    assert np.isnan(Or).all() and np.isnan(Wr).all()
    assert torch.isnan(O1[0]).all() and torch.isnan(W1[0]).all()
    G[17, 401] = 0.0
    W2, M2, O2 = run_step([W], [Mp], [G], 0.95, 0.02, 0.0, variant)
    Wr, Mr, Or = orc.muon_step(syn.to_f64(W), syn.to_f64(Mp), syn.to_f64(G), float(np.float32(0.95)),
                               float(np.float32(0.02)), 0.0, variant, state_dtype="bf16", w_dtype="f64")
    assert np.array_equal(syn.to_f64(M2[0]), Mr)
    assert relF(syn.to_f64(O2[0]), Or) < 2e-2


def test_bf16_output():
    M = syn.random_matrix(21, 256, 512, dtype="bf16")
    got = gpu_orth("standard", [M], "bf16", odt=torch.bfloat16)[0]
    assert relF(got, oracle_orth("standard", M)) < 2e-2


# ------------------------------------------------------------------ the Muon step
def run_step(Ws, Ms, Gs, mu_, lr, wd, variant, compute=None, O=True):
    W = [w.to(DEV) for w in Ws]
    M = [m.to(DEV) for m in Ms]
    G = [g.to(DEV) for g in Gs]
    Oo = [torch.empty(w.shape, dtype=torch.float32, device=DEV) for w in Ws] if O else None
    cfg = mu.NSConfig(compute=compute)
    mu.muon_step(W, M, G, mu_, lr, wd, variant, cfg, O_out=Oo)
    torch.cuda.synchronize()
    return [w.cpu() for w in W], [m.cpu() for m in M], ([o.cpu() for o in Oo] if O else None)


@pytest.mark.parametrize("variant,compute", [("standard", "f32"), ("standard", "bf16"), ("gram", "f16"), ("gram", "f32")])
def test_muon_step_single_256x512(variant, compute):
    wl = syn.WORKLOADS["single-256x512"]
    W, M, G = syn.matrix_inputs(wl, 0, 256, 512)
    mu_, lr, wd = 0.95, 0.02, 0.0
    W1, M1, O1 = run_step([W], [M], [G], mu_, lr, wd, variant, compute)
    mu32, lr32 = float(np.float32(mu_)), float(np.float32(lr))
    Wr, Mr, Or = orc.muon_step(syn.to_f64(W), syn.to_f64(M), syn.to_f64(G), mu32, lr32, wd, variant,
                               state_dtype="f32", w_dtype="f64")
    assert np.array_equal(syn.to_f64(M1[0]), Mr)
    tol = TOL[compute]
    assert relF(syn.to_f64(O1[0]), Or) < tol
    dW = syn.to_f64(W1[0]) - syn.to_f64(W)
    assert relF(dW, Wr - syn.to_f64(W)) < tol + 1e-4


@pytest.mark.parametrize("variant", ["standard", "gram"])
def test_muon_step_three_steps_bf16_state(variant):
    """llama-130m shapes, bf16 momentum, three consecutive steps from M = 0."""
    wl = syn.WORKLOADS["llama-130m"]
    Ws, Ms, _ = syn.group_inputs(wl, 1, count=2)
    Wg = [w.to(DEV) for w in Ws]
    Mg = [m.to(DEV) for m in Ms]
    Wo = [syn.to_f64(w) for w in Ws]
    Mo = [syn.to_f64(m) for m in Ms]
    mu32, lr32, wd = float(np.float32(0.95)), float(np.float32(0.02)), 0.01
    wd32 = float(np.float32(wd))
    for step in range(3):
        _, _, Gs = syn.group_inputs(wl, 1, count=2, step=step)
        Oo = [torch.empty(w.shape, dtype=torch.float32, device=DEV) for w in Ws]
        mu.muon_step(Wg, Mg, [g.to(DEV) for g in Gs], 0.95, 0.02, wd, variant, None, O_out=Oo)
        torch.cuda.synchronize()
        for i in range(2):
            Wn, Mn, On = orc.muon_step(Wo[i], Mo[i], syn.to_f64(Gs[i]), mu32, lr32, wd32, variant,
                                       state_dtype="bf16", w_dtype="f64")
            assert np.array_equal(syn.to_f64(Mg[i]), Mn), (step, i)
            assert relF(syn.to_f64(Oo[i]), On) < 2e-2
            dW = syn.to_f64(Wg[i]) - Wo[i]
            assert relF(dW, Wn - Wo[i]) < 2e-2 + 1e-3
            # continue the oracle from the GPU's weights so errors do not compound
            Wo[i] = syn.to_f64(Wg[i])
            Mo[i] = Mn


def test_muon_step_transposed_bf16_weights():
    r, c = 640, 256
    W = syn.random_matrix(30, r, c, dtype="bf16")
    M = torch.zeros(r, c, dtype=torch.bfloat16)
    G = syn.random_matrix(31, r, c, std=1e-3, dtype="bf16")
    W1, M1, O1 = run_step([W], [M], [G], 0.9, 0.05, 0.1, "standard")
    Wr, Mr, Or = orc.muon_step(syn.to_f64(W), syn.to_f64(M), syn.to_f64(G), float(np.float32(0.9)),
                               float(np.float32(0.05)), float(np.float32(0.1)), "standard",
                               state_dtype="bf16", w_dtype="f64")
    assert np.array_equal(syn.to_f64(M1[0]), Mr)
    assert relF(syn.to_f64(O1[0]), Or) < 2e-2
    # bf16 weights: the update is within the O tolerance plus one bf16 rounding
    err = np.abs(syn.to_f64(W1[0]) - Wr)
    assert np.all(err <= 0.05 * np.abs(syn.to_f64(O1[0]) - Or) + np.abs(Wr) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("variant", ["standard", "gram"])
@pytest.mark.parametrize("shape,w_bf16", [((300, 1100), False), ((1100, 300), True), ((512, 1536), True),
                                          ((768, 512), False)])
def test_last_product_same_update_for_every_output_choice(variant, shape, w_bf16):
    """The last product updates W from its fp32 result staged on chip, so W
    and M come out bit for bit the same whether O is also written (fp32 or
    bf16) or not, and the bf16 O is the fp32 O rounded to nearest even.  This
    covers each (W, O) dtype pair of the fused update, both orientations and
    ragged edges; the run without O (the usual training call) is also checked
    against the oracle."""
    r, c = shape
    W0 = syn.random_matrix(70, r, c, dtype="bf16" if w_bf16 else "f32")
    M0 = syn.random_matrix(71, r, c, std=1e-3, dtype="bf16")
    G0 = syn.random_matrix(72, r, c, std=1e-3, dtype="bf16")
    res = {}
    for odt in (None, torch.float32, torch.bfloat16):
        W, M, G = W0.to(DEV), M0.to(DEV), G0.to(DEV)
        O = None if odt is None else [torch.empty(r, c, dtype=odt, device=DEV)]
        mu.muon_step([W], [M], [G], 0.95, 0.02, 0.01, variant, None, O_out=O)
        torch.cuda.synchronize()
        res[odt] = (W.cpu(), M.cpu(), None if O is None else O[0].cpu())
    for odt in (torch.float32, torch.bfloat16):
        assert torch.equal(res[odt][0], res[None][0]) and torch.equal(res[odt][1], res[None][1]), odt
    assert torch.equal(res[torch.bfloat16][2], res[torch.float32][2].to(torch.bfloat16))
    mu32, lr32, wd32 = (float(np.float32(v)) for v in (0.95, 0.02, 0.01))
    Wr, Mr, Or = orc.muon_step(syn.to_f64(W0), syn.to_f64(M0), syn.to_f64(G0), mu32, lr32, wd32, variant,
                               state_dtype="bf16", w_dtype="f64")
    assert np.array_equal(syn.to_f64(res[None][1]), Mr)
    assert relF(syn.to_f64(res[torch.float32][2]), Or) < 2e-2
    dW = syn.to_f64(res[None][0]) - syn.to_f64(W0)
    # bf16 weights: the update also carries one bf16 rounding of W per element
    bound = 2e-2 + (np.abs(syn.to_f64(W0)).max() * 2.0 ** -8 * np.sqrt(r * c) / np.linalg.norm(Wr - syn.to_f64(W0))
                    if w_bf16 else 1e-4)
    assert relF(dW, Wr - syn.to_f64(W0)) < bound


@pytest.mark.parametrize("variant,compute", [("standard", "bf16"), ("gram", "f16"), ("standard", "f32")])
@pytest.mark.parametrize("shape", [(256, 700), (300, 200)])
def test_muon_step_update_scale_and_weight_decay(variant, compute, shape):
    """W <- W - lr (s O + wd W): against the GPU's own O elementwise (fp32
    arithmetic), against the oracle at the O tolerance, and s = 1 is the
    default call bit for bit."""
    r, c = shape
    W = syn.random_matrix(40, r, c)
    M = syn.random_matrix(41, r, c, std=1e-3, dtype="bf16")
    G = syn.random_matrix(42, r, c, std=1e-3, dtype="bf16")
    mu_, lr, wd, s = 0.9, 0.05, 0.1, 0.37
    cfg = mu.NSConfig(compute=compute)

    def step(scale):
        Wg, Mg = [W.to(DEV)], [M.to(DEV)]
        Oo = [torch.empty(r, c, dtype=torch.float32, device=DEV)]
        kw = {} if scale is None else {"update_scale": scale}
        mu.muon_step(Wg, Mg, [G.to(DEV)], mu_, lr, wd, variant, cfg, O_out=Oo, **kw)
        torch.cuda.synchronize()
        return Wg[0].cpu(), Mg[0].cpu(), Oo[0].cpu()

    W1, M1, O1 = step(s)
    f32 = np.float32
    ref32 = torch.from_numpy((W.numpy() - f32(lr) * (f32(s) * O1.numpy() + f32(wd) * W.numpy())).astype(np.float32))
    torch.testing.assert_close(W1, ref32, rtol=2e-7, atol=2e-7)
    Wr, Mr, Or = orc.muon_step(syn.to_f64(W), syn.to_f64(M), syn.to_f64(G), float(f32(mu_)), float(f32(lr)),
                               float(f32(wd)), variant, state_dtype="bf16", w_dtype="f64",
                               update_scale=float(f32(s)))
    assert np.array_equal(syn.to_f64(M1), Mr)
    assert relF(syn.to_f64(O1), Or) < TOL[compute]
    dW = syn.to_f64(W1) - syn.to_f64(W)
    assert relF(dW, Wr - syn.to_f64(W)) < TOL[compute] + 1e-4
    Wa, _, _ = step(1.0)
    Wb, _, _ = step(None)
    assert torch.equal(Wa, Wb)


def test_checkpoint_resume_is_bitwise():
    """Two steps straight equal one step, a copy of (W, M), and one more step."""
    wl = syn.WORKLOADS["llama-130m"]
    Ws, Ms, G0 = syn.group_inputs(wl, 0, count=1, step=0)
    _, _, G1 = syn.group_inputs(wl, 0, count=1, step=1)
    Wa, Ma = [Ws[0].to(DEV)], [Ms[0].to(DEV)]
    for G in (G0, G1):
        mu.muon_step(Wa, Ma, [G[0].to(DEV)], 0.95, 0.02, 0.0, "gram")
    Wb, Mb = [Ws[0].to(DEV)], [Ms[0].to(DEV)]
    mu.muon_step(Wb, Mb, [G0[0].to(DEV)], 0.95, 0.02, 0.0, "gram")
    Wc, Mc = [Wb[0].cpu().clone().to(DEV)], [Mb[0].cpu().clone().to(DEV)]
    mu.muon_step(Wc, Mc, [G1[0].to(DEV)], 0.95, 0.02, 0.0, "gram")
    torch.cuda.synchronize()
    assert torch.equal(Wa[0], Wc[0]) and torch.equal(Ma[0], Mc[0])


@pytest.mark.parametrize("variant", ["standard", "gram"])
def test_muon_step_in_a_hip_graph(variant):
    """The step launches kernels only (no memsets or copies on the stream), so
    it can be captured in a HIP graph: each of several replays, with eager work
    and synchronisations in between, equals the same step run eagerly."""
    wl = syn.WORKLOADS["llama-130m"]
    Ws, Ms, Gs = syn.group_inputs(wl, 1, count=3)
    Wg, Mg, Gg = [w.to(DEV) for w in Ws], [m.to(DEV) for m in Ms], [g.to(DEV) for g in Gs]
    We, Me = [w.clone() for w in Wg], [m.clone() for m in Mg]
    ws = torch.empty(mu.workspace_size(3, *Ws[0].shape, variant), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (caches the pointer arrays)
        Wt, Mt = [w.clone() for w in Wg], [m.clone() for m in Mg]
        mu.muon_step(Wt, Mt, Gg, 0.95, 0.02, 0.01, variant, None, workspace=ws)
        mu.muon_step(Wg, Mg, Gg, 0.95, 0.02, 0.01, variant, None, workspace=ws)  # pointers used in the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mu.muon_step(We, Me, Gg, 0.95, 0.02, 0.01, variant, None)  # eager copy of the same first step
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(Wg, We)) and all(torch.equal(a, b) for a, b in zip(Mg, Me))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mu.muon_step(Wg, Mg, Gg, 0.95, 0.02, 0.01, variant, None, workspace=ws)
    for rep in range(3):
        g.replay()
        junk = torch.randn(1 << 20, device=DEV).sum()  # the program's own eager work between replays
        mu.muon_step(We, Me, Gg, 0.95, 0.02, 0.01, variant, None)
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for a, b in zip(Wg, We):
            assert torch.equal(a, b), rep
        for a, b in zip(Mg, Me):
            assert torch.equal(a, b), rep


def test_capture_without_a_prior_call_raises_cleanly():
    """Pointer arrays are made by a host-to-device copy, which a capturing
    stream does not allow: capturing a step on tensors never used before
    raises MuonError before anything is enqueued, and the device stays usable
    (a normal step afterwards matches one on a copy of the inputs)."""
    W = [syn.random_matrix(80, 256, 512).to(DEV)]
    M = [torch.zeros(256, 512, dtype=torch.bfloat16, device=DEV)]
    G = [syn.random_matrix(81, 256, 512, std=1e-3, dtype="bf16").to(DEV)]
    ws = torch.empty(mu.workspace_size(1, 256, 512, "gram"), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    # the allocator may hand out addresses an earlier test's arrays were keyed on
    from matrix_orthogonalizing_optimizer_step_amd import binding as bd
    for lst in (W, M, G):
        key = (str(lst[0].device), tuple(int(t.data_ptr()) for t in lst))
        bd._ptr_cache.pop(key, None)
        bd._ptr_pinned.pop(key, None)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(mu.MuonError, match="before capturing"):
        with torch.cuda.graph(g):
            mu.muon_step(W, M, G, 0.95, 0.02, 0.0, "gram", None, workspace=ws)
    We, Me = [w.clone() for w in W], [m.clone() for m in M]
    mu.muon_step(W, M, G, 0.95, 0.02, 0.0, "gram", None, workspace=ws)
    mu.muon_step(We, Me, G, 0.95, 0.02, 0.0, "gram", None)
    torch.cuda.synchronize()
    assert torch.equal(W[0], We[0]) and torch.equal(M[0], Me[0])


@pytest.mark.parametrize("variant", ["standard", "gram"])
def test_narrow_and_wide_tiles_agree_bitwise(variant):
    """A batch of one 512x1536 matrix runs its symmetric products in 256x128
    tiles (3 tiles of 256x256 leave the last round nearly empty) and a batch
    of 43 runs them in 256x256 tiles (129 tiles); every output element sums
    the same k-steps in the same order, so without the trace shift (whose
    per-tile partials are grouped differently) the first matrix's result is
    the same bit for bit."""
    Ms = [syn.random_matrix(60 + i, 512, 1536, std=1e-3, dtype="bf16") for i in range(43)]
    cfg = mu.NSConfig(shift=False)
    f = mu.ns_orthogonalize if variant == "standard" else mu.gram_ns_orthogonalize
    outs = []
    for batch in (Ms[:1], Ms):
        O = [torch.empty(512, 1536, device=DEV) for _ in batch]
        f([m.to(DEV) for m in batch], O, cfg)
        torch.cuda.synchronize()
        outs.append(O[0].cpu())
    assert torch.equal(outs[0], outs[1])
    ref = oracle_orth(variant, Ms[0])
    assert relF(syn.to_f64(outs[0]), ref) < 2e-2


def test_fresh_tensors_make_no_host_stall_and_streams_stay_ordered():
    """A step on tensors never seen before builds its pointer arrays with an
    asynchronous copy: with the stream busy for a while, building them
    returns at once (the host does not wait for the device).  Steps with
    fresh gradients alternating between two streams, with no host
    synchronisation, equal the same steps run on one stream."""
    import time

    from matrix_orthogonalizing_optimizer_step_amd import binding as bd
    r, c = 300, 520
    busy = torch.randn(4096, 4096, device=DEV)
    torch.cuda.synchronize()
    for _ in range(40):  # about 0.1 s of work queued on the current stream
        busy = (busy @ busy) * 1e-4
    fresh = [torch.empty(r, c, device=DEV) for _ in range(3)]
    t0 = time.perf_counter()
    arr = bd.pointer_array(fresh)
    dt = time.perf_counter() - t0
    still_busy = not torch.cuda.current_stream().query()
    torch.cuda.synchronize()
    assert arr.cpu().tolist() == [t.data_ptr() for t in fresh]
    assert still_busy and dt < 0.03, (still_busy, dt)

    W0 = syn.random_matrix(97, r, c)
    Gs = [syn.random_matrix(98 + i, r, c, std=1e-3, dtype="bf16") for i in range(4)]
    side = torch.cuda.Stream()
    Wa, Ma = [W0.to(DEV)], [torch.zeros(r, c, dtype=torch.bfloat16, device=DEV)]
    Wb, Mb = [W0.to(DEV)], [torch.zeros(r, c, dtype=torch.bfloat16, device=DEV)]
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    fresh_a = [G.to(DEV) for G in Gs]  # kept alive to the end: each step sees new addresses
    fresh_b = [G.to(DEV) for G in Gs]
    torch.cuda.synchronize()
    for i in range(len(Gs)):
        s = side if i % 2 else main
        s.wait_stream(main if i % 2 else side)
        with torch.cuda.stream(s):
            mu.muon_step(Wa, Ma, [fresh_a[i]], 0.95, 0.02, 0.0, "gram")
        mu.muon_step(Wb, Mb, [fresh_b[i]], 0.95, 0.02, 0.0, "gram")
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(Wa[0], Wb[0]) and torch.equal(Ma[0], Mb[0])


@pytest.mark.parametrize("mu_", [0.5, 0.95])
def test_momentum_rounding_ties_and_extremes(mu_):
    """The momentum M <- mu M + G is rounded once to bf16, bit for bit as the
    oracle rounds the exact value: on exact ties and values just either side
    of them (mu = 0.5 makes mu M exact, so M + G can sit exactly half-way
    between two bf16 values), on bf16 subnormals (below 2^-126), near the
    largest bf16 value and on overflow to infinity."""
    r = np.random.default_rng(77)
    n = 64 * 96
    g = orc.round_bf16(r.standard_normal(n) * 2.0 ** r.integers(-20, 20, n))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(g))) - 7)
    kind = r.integers(0, 6, n)
    # mu m lands at ulp/2 (a tie), or one step of m either side of it
    m = np.where(kind == 0, ulp, np.where(kind == 1, ulp * (1 + 2.0 ** -7), ulp * (1 - 2.0 ** -8))) / (2 * mu_)
    m = orc.round_bf16(m * np.where(r.random(n) < 0.5, -1.0, 1.0))
    # bf16 subnormals and tiny values, huge values and overflow
    m[kind == 3] = orc.round_bf16(r.standard_normal((kind == 3).sum()) * 2.0 ** -130)
    g[kind == 3] = orc.round_bf16(r.standard_normal((kind == 3).sum()) * 2.0 ** -128)
    k4 = (kind == 4).sum()
    m[kind == 4] = orc.round_bf16(3.0e38 * np.sign(r.standard_normal(k4)))
    g[kind == 4] = orc.round_bf16(3.0e38 * r.uniform(-1.0, 1.0, k4))  # same sign: overflow; opposite: near the top
    # bf16 tensors made from their bit patterns: a host conversion may flush
    # bf16 subnormals to zero
    def to_bf16(x):
        bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return torch.from_numpy(bits.view(np.int16).reshape(64, 96)).view(torch.bfloat16)

    def from_bf16(t):
        bits = t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64).ravel()

    M, G = to_bf16(m), to_bf16(g)
    assert np.array_equal(from_bf16(M), m) and np.array_equal(from_bf16(G), g)
    W = torch.zeros(64, 96)
    _, M1, _ = run_step([W], [M], [G], mu_, 0.0, 0.0, "standard", O=False)
    want = orc.round_bf16(float(np.float32(mu_)) * m + g)
    got = from_bf16(M1[0])
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:8]
    assert np.isinf(want).any() and (np.abs(want[np.isfinite(want) & (want != 0)]) < 2.0 ** -126).any()
    if mu_ == 0.5:  # exact ties are present
        x = mu_ * m + g
        assert (np.abs(x - want) == ulp / 2).sum() > 100
