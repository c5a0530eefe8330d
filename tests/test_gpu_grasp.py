"""GPU parity of the low-bit momentum state (through the C ABI) against the
fp64 oracle in oracle/grasp_oracle.py.

* The two codes on their own are bit-exact: the same fp32 input gives the
  same codes and scales, and decoding gives the fp32 rounding of the
  oracle's fp64 value.
* k = 0 (no subspace): M_t and the new 4-bit state are bit-exact.
* k > 0: M_t from a given state agrees to fp32 rounding; the power
  iteration's P and R (8-bit) and the residual (4-bit) are computed from
  products near fp32 accuracy on the GPU and in fp64 by the oracle, so a code
  may differ by one where the oracle's unrounded value L x / m lies near a
  rounding boundary.  The Q factor of M_t Q moves by about cond(M_t Q) times
  the relative error of the product (a property of QR, not of the method used),
  so the reach grows with the conditioning: the test allows a 1 % share of
  codes that differ by one, each within 0.75 of the oracle's unrounded value
  (one of the two nearest codes), and compares the decoded state and O at
  relative Frobenius error.
"""
import numpy as np
import pytest
import torch

import matrix_orthogonalizing_optimizer_step_amd as mu
from oracle import grasp_oracle as go
from oracle import muon_oracle as orc
from synth import inputs as syn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MU, LR = float(np.float32(0.95)), float(np.float32(0.02))


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def host(t):
    return t.detach().cpu().numpy()


def seeded(seed, rows, cols, std=1.0):
    return syn.to_f64(syn.random_matrix(seed, rows, cols, std)).astype(np.float32)


# ------------------------------------------------------------ the codes alone
@pytest.mark.parametrize("rows,cols", [(130, 260), (1, 1), (257, 3), (128, 128), (3, 515)])
def test_grid_code_bitexact(rows, cols):
    x = seeded(rows * 7 + cols, rows, cols)
    x[::5, ::3] *= 40  # two-sided outliers
    if rows >= 128 and cols >= 128:
        x[:64, :64] = 0                                    # a zero corner of a block
        x[100, 7] = np.float32(3.0) * np.abs(x[100]).max()  # a row/column extreme
    q, sr, sc = go.grid_quantize(x)
    codes, gsr, gsc = mu.grid_quantize([dev(x)])
    torch.cuda.synchronize()
    assert np.array_equal(host(codes[0]), go.pack_nibbles(q))
    assert np.array_equal(host(gsr[0]), sr) and np.array_equal(host(gsc[0]), sc)
    y = mu.grid_dequantize(codes, gsr, gsc, cols)
    torch.cuda.synchronize()
    assert np.array_equal(host(y[0]), go.grid_dequantize(q, sr, sc).astype(np.float32))


def test_grid_code_ties_nan_inf():
    m = np.float32(1.75)
    x = np.zeros((3, 6), np.float32)
    x[0, :4] = [m, m / 2, np.float32(5 * 1.75 / 14), -m / 2]
    x[1, :4] = m
    x[2, 4] = np.nan
    x[0, 5] = np.inf
    q, sr, sc = go.grid_quantize(x)
    codes, gsr, gsc = mu.grid_quantize([dev(x)])
    torch.cuda.synchronize()
    assert list(q[0, :4]) == [7, 4, 2, -4]
    assert np.array_equal(host(codes[0]), go.pack_nibbles(q))
    np.testing.assert_array_equal(host(gsr[0]), sr)  # NaN in the same places
    np.testing.assert_array_equal(host(gsc[0]), sc)


@pytest.mark.parametrize("rows,k", [(300, 224), (5, 1), (17, 300), (64, 128)])
def test_group8_code_bitexact(rows, k):
    x = seeded(rows + 11 * k, rows, k)
    x[:, ::7] *= 30
    q, s = go.group8_quantize(x)
    codes, scales = mu.group8_quantize([dev(x)])
    torch.cuda.synchronize()
    assert np.array_equal(host(codes[0]), q) and np.array_equal(host(scales[0]), s)
    y = mu.group8_dequantize(codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(host(y[0]), go.group8_dequantize(q, s).astype(np.float32))


# ------------------------------------------------------------ helpers for the step
def gpu_state_from(st, rows, cols, k):
    """Device copy of an oracle-layout state (codes unpacked -> packed bytes)."""
    gs = mu.GraspState(1, rows, cols, 0, DEV)
    gs.k = k
    gs.res_codes = [dev(go.pack_nibbles(st["res_codes"]))]
    gs.res_row_scales = [dev(st["res_sr"])]
    gs.res_col_scales = [dev(st["res_sc"])]
    if k > 0:
        gs.P_codes, gs.P_scales = [dev(st["P_codes"])], [dev(st["P_scales"])]
        gs.R_codes, gs.R_scales = [dev(st["R_codes"])], [dev(st["R_scales"])]
    return gs


def random_state(seed, rows, cols, k, res_scale=0.1, f_scale=0.05):
    """An arbitrary valid state from seeded random codes and scales."""
    nb = lambda n: (n + 127) // 128  # noqa: E731
    st = dict(res_codes=syn.random_codes(seed, (rows, cols), 7),
              res_sr=syn.random_scales(seed + 1, (rows, nb(cols)), res_scale),
              res_sc=syn.random_scales(seed + 2, (nb(rows), cols), res_scale))
    if k > 0:
        st["P_codes"] = syn.random_codes(seed + 3, (rows, k), 127)
        st["P_scales"] = syn.random_scales(seed + 4, (rows, nb(k)), f_scale)
        st["R_codes"] = syn.random_codes(seed + 5, (cols, k), 127)
        st["R_scales"] = syn.random_scales(seed + 6, (cols, nb(k)), f_scale)
    return st


def near_tie_mismatch(q_gpu, q_or, x_or, m, levels, share=0.01, reach=0.75):
    """Codes equal except a small share that differ by one, each of them
    within ``reach`` of the oracle's unrounded L x / m (one of the two codes
    nearest to the exact value)."""
    q_gpu = q_gpu.astype(np.int32)
    q_or = q_or.astype(np.int32)
    diff = q_gpu != q_or
    if not diff.any():
        return 0.0
    assert np.abs(q_gpu - q_or).max() == 1
    t = levels * np.asarray(x_or, np.float64)[diff] / np.asarray(m, np.float64)[diff]
    assert np.all(np.abs(t - q_gpu[diff]) < reach), "a code differs away from a rounding boundary"
    frac = diff.mean()
    assert frac <= share, frac
    return frac


def close_scales(got, want):
    """Scales (largest magnitudes) agree to the products' accuracy: relative
    2e-3, or 1e-3 of the matrix's largest scale (a residual of a momentum with
    a strong top subspace is small, and its error is set by the size of M_t;
    a CPU emulation of the split-bf16 products reproduces the GPU's figures)."""
    np.testing.assert_allclose(got, want, rtol=2e-3, atol=1e-3 * float(np.abs(want).max()))


def compare_state(gs, st, det, rows, cols, k, M_ref=None):
    """The new state against the oracle's.  When M_t lies in the subspace
    (k = rank: the oracle's residual is fp64 rounding noise, the GPU's is the
    products' rounding noise), the residual's codes are noise on both sides:
    then only its size is checked, against M_t."""
    torch.cuda.synchronize()
    q_gpu = go.unpack_nibbles(host(gs.res_codes[0]), cols)
    sr, sc = host(gs.res_row_scales[0]), host(gs.res_col_scales[0])
    rec_gpu = go.grid_dequantize(q_gpu, sr, sc)
    f_res = 0.0
    if M_ref is not None and np.linalg.norm(det["M_res"]) <= 1e-6 * np.linalg.norm(M_ref):
        assert np.linalg.norm(rec_gpu) <= 1e-4 * np.linalg.norm(M_ref)
    else:
        close_scales(sr, st["res_sr"])
        close_scales(sc, st["res_sc"])
        m_or = go.grid_min_scale(st["res_sr"], st["res_sc"], rows, cols)
        f_res = near_tie_mismatch(q_gpu, st["res_codes"], det["M_res"], m_or, 7)
    rec_or = go.grid_dequantize(st["res_codes"], st["res_sr"], st["res_sc"])
    if k > 0:
        for name, key in (("P", "P"), ("R", "R")):
            qg, sg = host(getattr(gs, name + "_codes")[0]), host(getattr(gs, name + "_scales")[0])
            close_scales(sg, st[name + "_scales"])
            mo_ = np.repeat(st[name + "_scales"], 128, axis=1)[:, :k]
            near_tie_mismatch(qg, st[name + "_codes"], det[key].astype(np.float32), mo_, 127)
        Pg = go.group8_dequantize(host(gs.P_codes[0]), host(gs.P_scales[0]))
        Rg = go.group8_dequantize(host(gs.R_codes[0]), host(gs.R_scales[0]))
        Po = go.group8_dequantize(st["P_codes"], st["P_scales"])
        Ro = go.group8_dequantize(st["R_codes"], st["R_scales"])
        rec_gpu = rec_gpu + Pg @ Rg.T
        rec_or = rec_or + Po @ Ro.T
    assert orc.relative_frobenius(rec_gpu, rec_or) < 1e-2
    return f_res


def run_both(W, st_or, gs, G, k, variant, M_out=True, aux=False):
    rows, cols = G.shape
    Wd, Gd = [dev(W)], [dev(G)]
    O = [torch.empty(rows, cols, dtype=torch.float32, device=DEV)]
    Mt = [torch.empty(rows, cols, dtype=torch.float32, device=DEV)] if M_out else None
    mu.grasp_step(Wd, gs, Gd, MU, LR, 0.0, variant, O_out=O, M_out=Mt,
                  aux_stream=torch.cuda.Stream() if aux else None)
    torch.cuda.synchronize()
    W1, st1, O1, M1, det = go.grasp_step(W.astype(np.float64), st_or, G, MU, LR, 0.0, variant)
    return (host(Wd[0]), host(O[0]), host(Mt[0]) if M_out else None), (W1, st1, O1, M1, det)


# ------------------------------------------------------------ the step
@pytest.mark.parametrize("rows,cols", [(300, 520), (520, 300), (129, 1)])
def test_grasp_step_without_subspace_bitexact(rows, cols):
    """k = 0, two steps from the zero state: M_t and the state bit for bit."""
    st = go.new_state(rows, cols, 0)
    gs = mu.GraspState(1, rows, cols, 0, DEV)
    W = seeded(1, rows, cols)
    for step in range(2):
        G = seeded(10 + step, rows, cols, 0.01)
        (Wg, Og, Mg), (W1, st, O1, M1, det) = run_both(W, st, gs, G, 0, "standard")
        assert np.array_equal(Mg, M1.astype(np.float32)), step
        assert np.array_equal(go.unpack_nibbles(host(gs.res_codes[0]), cols), st["res_codes"])
        assert np.array_equal(host(gs.res_row_scales[0]), st["res_sr"])
        assert np.array_equal(host(gs.res_col_scales[0]), st["res_sc"])
        if min(rows, cols) > 1:
            assert orc.relative_frobenius(Og, O1) < 2e-2
        assert orc.relative_frobenius(Wg - W, W1 - W) < 2e-2 + 1e-4


@pytest.mark.parametrize("aux", [False, True], ids=["one-stream", "aux-stream"])
@pytest.mark.parametrize("rows,cols,k,variant", [
    (300, 520, 20, "standard"),
    (520, 300, 20, "gram"),
    (384, 640, 130, "standard"),   # two 8-bit groups per row of P and R
    (256, 4096, 16, "gram"),      # M_t Q split along k
    (4096, 256, 16, "standard"),  # M_t^T P split along k
    (200, 150, 1, "standard"),
    (600, 700, 300, "gram"),      # k > 256: the panel Cholesky (16-row panels), 3 groups
    (300, 520, 256, "standard"),  # the largest k of the register-resident Cholesky: every slot block in use
    (400, 300, 255, "gram"),      # k odd, next to that limit, iterated transposed
    (270, 300, 257, "standard"),  # the smallest k of the panel Cholesky
    (700, 1100, 520, "standard"), # the blocked solve's X rows beyond 64 KB of LDS, 5 groups
    (1100, 1030, 1024, "gram"),   # the largest k, iterated transposed
    (257, 1, 1, "standard"),      # a column: k = min(rows, cols) = 1
    (1, 300, 1, "gram"),          # a row
])
def test_grasp_step_from_a_random_state(rows, cols, k, variant, aux):
    """One step from an arbitrary state: M_t to fp32 rounding, the new state
    up to near-tie codes, O and W at the 16-bit tolerance; with an aux stream
    the state update runs beside Newton-Schulz and must give the same."""
    st = random_state(rows + cols + k, rows, cols, k)
    gs = gpu_state_from(st, rows, cols, k)
    W = seeded(2, rows, cols)
    G = seeded(3, rows, cols, 0.01)
    (Wg, Og, Mg), (W1, st1, O1, M1, det) = run_both(W, st, gs, G, k, variant, aux=aux)
    err = np.abs(Mg.astype(np.float64) - M1)
    assert np.all(err <= 1.2e-7 * np.abs(M1) + 1e-12 * np.abs(M1).max())
    f = compare_state(gs, st1, det, rows, cols, k, M_ref=M1)
    assert orc.relative_frobenius(Og, O1) < 2e-2
    assert orc.relative_frobenius(Wg - W, W1 - W) < 2e-2 + 1e-4
    print(f"{rows}x{cols} k={k} {variant}: residual codes off by one {f:.2e}")


def test_grasp_first_steps_with_a_low_rank_momentum():
    """From the start state (zero residual and P, Gaussian R): two steps on a
    gradient of rank k plus noise; after the warm-started second step the
    subspace holds the low-rank part, the residual is small and the decoded
    state tracks M_t."""
    rows, cols, k = 320, 448, 12
    U = seeded(20, rows, k)
    V = seeded(21, k, cols)
    R0 = seeded(22, cols, k)
    st = go.new_state(rows, cols, k, R_init=R0)
    gs = mu.GraspState(1, rows, cols, k, DEV, R_init=[dev(R0)])
    torch.cuda.synchronize()
    assert np.array_equal(host(gs.R_codes[0]), st["R_codes"]) and np.array_equal(host(gs.R_scales[0]), st["R_scales"])
    W = seeded(23, rows, cols)
    for step in range(2):
        G = (U @ V + 0.05 * seeded(30 + step, rows, cols)).astype(np.float32)
        (Wg, Og, Mg), (W1, st_next, O1, M1, det) = run_both(W, st, gs, G, k, "gram")
        if step == 0:
            assert np.array_equal(Mg, M1.astype(np.float32))  # M_{-1} = 0
            compare_state(gs, st_next, det, rows, cols, k)
        else:
            # each side now runs on its own state, so the two M_t differ by the
            # near-tie codes of step 0: compare the two M_t, and what each side
            # stored with its own M_t
            assert orc.relative_frobenius(Mg, M1) < 1e-2
            torch.cuda.synchronize()
            rec_g = go.grid_dequantize(go.unpack_nibbles(host(gs.res_codes[0]), cols), host(gs.res_row_scales[0]),
                                       host(gs.res_col_scales[0])) + \
                go.group8_dequantize(host(gs.P_codes[0]), host(gs.P_scales[0])) @ \
                go.group8_dequantize(host(gs.R_codes[0]), host(gs.R_scales[0])).T
            rec_o = go.reconstruct(st_next)
            assert orc.relative_frobenius(rec_g, Mg) < 2e-2 and orc.relative_frobenius(rec_o, M1) < 2e-2
        # a cold start (random R) leaves about a fifth; the warm start about 1 %
        assert np.linalg.norm(det["M_res"]) < (0.3 if step == 0 else 0.03) * np.linalg.norm(M1)
        if step == 0:  # later, O = NS(M_t) magnifies the small state differences in the weak directions
            assert orc.relative_frobenius(Og, O1) < 2e-2
        st = st_next  # each side keeps its own state; W is the same seeded matrix every step


def test_grasp_zero_column_of_R():
    """A zero column of R_{t-1} gives a zero column of Q, hence of P and R."""
    rows, cols, k = 160, 200, 6
    st = random_state(77, rows, cols, k)
    st["R_codes"][:, 3] = 0
    gs = gpu_state_from(st, rows, cols, k)
    G = seeded(5, rows, cols, 0.01)
    (Wg, Og, Mg), (W1, st1, O1, M1, det) = run_both(seeded(6, rows, cols), st, gs, G, k, "standard")
    assert np.all(host(gs.P_codes[0])[:, 3] == 0) and np.all(st1["P_codes"][:, 3] == 0)
    assert np.all(host(gs.R_codes[0])[:, 3] == 0)
    compare_state(gs, st1, det, rows, cols, k)


@pytest.mark.parametrize("rows,cols,k", [(200, 300, 20), (300, 250, 224)], ids=["k20", "k224-transposed"])
def test_grasp_all_zero_momentum(rows, cols, k):
    """A zero gradient on the zero state: M_t = 0, so P~ = M_t Q = 0, S = 0
    and every column of the Cholesky factor is dead (its diagonal entry is not
    positive), which the solve turns into P = 0; then R = 0, the residual and
    all codes are zero, O = 0 and W does not move, on both sides."""
    R_init = seeded(90, cols, k)
    st = go.new_state(rows, cols, k, R_init=R_init)
    gs = gpu_state_from(st, rows, cols, k)
    W = seeded(91, rows, cols)
    G = np.zeros((rows, cols), np.float32)
    (Wg, Og, Mg), (W1, st1, O1, M1, det) = run_both(W, st, gs, G, k, "gram")
    assert not np.any(M1) and not np.any(Mg)
    assert not np.any(det["P"]) and not np.any(O1) and not np.any(Og)
    for name in ("P_codes", "P_scales", "R_codes", "R_scales"):
        assert not np.any(st1[name]) and not np.any(host(getattr(gs, name)[0])), name
    assert not np.any(host(gs.res_codes[0])) and not np.any(host(gs.res_row_scales[0]))
    assert np.array_equal(Wg, W) and np.array_equal(W1.astype(np.float32), W)


@pytest.mark.parametrize("rows,cols,k", [(3584, 18944, 224), (3584, 512, 32)], ids=["qwen-mlp", "qwen-kv"])
def test_grasp_state_full_size(rows, cols, k):
    """Full-size matrices of the Qwen2.5-7B layer set at rank / 16, from a
    random state: M_t to fp32 rounding and the new state as in the smaller
    cases (the oracle computes the momentum and the state only; its fp64
    Newton-Schulz at this size would take minutes, and O is covered by the
    step tests above and by the full-size Newton-Schulz tests)."""
    st = random_state(rows // 7 + k, rows, cols, k)
    gs = gpu_state_from(st, rows, cols, k)
    G = seeded(40, rows, cols, 1e-3)
    Mt = [torch.empty(rows, cols, dtype=torch.float32, device=DEV)]
    mu.grasp_step([dev(seeded(41, rows, cols))], gs, [dev(G)], MU, LR, 0.0, "gram", M_out=Mt)
    torch.cuda.synchronize()
    Mg = host(Mt[0])
    M1 = go.momentum(st, G, MU)
    err = np.abs(Mg.astype(np.float64) - M1)
    assert np.all(err <= 1.2e-7 * np.abs(M1) + 1e-12 * np.abs(M1).max())
    st1, det = go.compress(M1, st)
    f = compare_state(gs, st1, det, rows, cols, k)
    print(f"{rows}x{cols} k={k}: residual codes off by one {f:.2e}")


@pytest.mark.parametrize("aux", [False, True], ids=["one-stream", "aux-stream"])
@pytest.mark.parametrize("k", [0, 12])
def test_grasp_step_in_a_hip_graph(k, aux):
    """The low-bit step also launches kernels only (no memsets or copies), so
    it can be captured once and replayed: each replay, with the program's own
    eager work and synchronisations between replays, advances the state
    exactly as an eager step does (bit for bit: every reduction has a fixed
    order)."""
    rows, cols = 320, 448
    R0 = [dev(seeded(50, cols, k))] if k else None
    sg = mu.GraspState(1, rows, cols, k, DEV, R_init=R0)
    se = mu.GraspState(1, rows, cols, k, DEV, R_init=R0)
    Wg = [dev(seeded(51, rows, cols))]
    We = [Wg[0].clone()]
    G = [dev(seeded(52, rows, cols, 0.01))]
    ws = torch.empty(mu.grasp_workspace_size(1, rows, cols, k, "gram"), dtype=torch.uint8, device=DEV)
    names = ["res_codes", "res_row_scales", "res_col_scales"] + (["P_codes", "P_scales", "R_codes", "R_scales"] if k else [])

    def same():
        torch.cuda.synchronize()
        assert torch.equal(Wg[0], We[0])
        for n in names:
            assert torch.equal(getattr(sg, n)[0], getattr(se, n)[0]), n

    ax = torch.cuda.Stream() if aux else None  # captured too: it joins the capture through the fork event
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (caches the pointer arrays)
        mu.grasp_step(Wg, sg, G, MU, LR, 0.0, "gram", workspace=ws, aux_stream=ax)
    torch.cuda.current_stream().wait_stream(side)
    mu.grasp_step(We, se, G, MU, LR, 0.0, "gram")
    same()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mu.grasp_step(Wg, sg, G, MU, LR, 0.0, "gram", workspace=ws, aux_stream=ax)
    for rep in range(3):
        g.replay()
        junk = torch.randn(1 << 20, device=DEV).sum()
        mu.grasp_step(We, se, G, MU, LR, 0.0, "gram")
        assert float(junk) == float(junk)
        same()


@pytest.mark.parametrize("rows,cols,k", [(300, 520, 20), (2048, 256, 16)], ids=["300x520-k20", "2048x256-k16"])
def test_grasp_step_batched(rows, cols, k):
    """A batch of 3 matrices in one call, each with its own random state:
    every matrix matches the oracle on its own (per-matrix pointers, strided
    workspace slices, split products over the batch)."""
    n = 3
    sts = [random_state(1000 + 37 * i + k, rows, cols, k) for i in range(n)]
    gs = mu.GraspState(n, rows, cols, 0, DEV)
    gs.k = k
    gs.res_codes = [dev(go.pack_nibbles(st["res_codes"])) for st in sts]
    gs.res_row_scales = [dev(st["res_sr"]) for st in sts]
    gs.res_col_scales = [dev(st["res_sc"]) for st in sts]
    gs.P_codes = [dev(st["P_codes"]) for st in sts]
    gs.P_scales = [dev(st["P_scales"]) for st in sts]
    gs.R_codes = [dev(st["R_codes"]) for st in sts]
    gs.R_scales = [dev(st["R_scales"]) for st in sts]
    Ws = [seeded(60 + i, rows, cols) for i in range(n)]
    Gs = [seeded(70 + i, rows, cols, 0.01) for i in range(n)]
    Wd = [dev(w) for w in Ws]
    O = [torch.empty(rows, cols, dtype=torch.float32, device=DEV) for _ in range(n)]
    Mt = [torch.empty(rows, cols, dtype=torch.float32, device=DEV) for _ in range(n)]
    mu.grasp_step(Wd, gs, [dev(g) for g in Gs], MU, LR, 0.0, "gram", O_out=O, M_out=Mt)
    torch.cuda.synchronize()
    for i in range(n):
        W1, st1, O1, M1, det = go.grasp_step(Ws[i].astype(np.float64), sts[i], Gs[i], MU, LR, 0.0, "gram")
        Mg = host(Mt[i])
        assert np.all(np.abs(Mg.astype(np.float64) - M1) <= 1.2e-7 * np.abs(M1) + 1e-12 * np.abs(M1).max()), i
        one = mu.GraspState(1, rows, cols, 0, DEV)
        one.k = k
        for name in ("res_codes", "res_row_scales", "res_col_scales", "P_codes", "P_scales", "R_codes", "R_scales"):
            setattr(one, name, [getattr(gs, name)[i]])
        compare_state(one, st1, det, rows, cols, k)
        assert orc.relative_frobenius(host(O[i]), O1) < 2e-2, i


def test_grasp_step_with_offset_buffers():
    """User buffers need not be aligned: a bf16 gradient two bytes off and a
    code buffer one byte off (views into larger allocations) take the
    element-wise paths and still give M_t and the state bit for bit."""
    rows, cols = 64, 256
    g = seeded(80, rows, cols, 0.01)
    gbuf = torch.empty(rows * cols + 1, dtype=torch.bfloat16, device=DEV)
    G = gbuf[1:].view(rows, cols)
    G.copy_(torch.from_numpy(g).to(DEV, torch.bfloat16))
    gs = mu.GraspState(1, rows, cols, 0, DEV)
    cbuf = torch.zeros(rows * cols // 2 + 1, dtype=torch.uint8, device=DEV)
    gs.res_codes = [cbuf[1:].view(rows, cols // 2)]
    Mt = [torch.empty(rows, cols, dtype=torch.float32, device=DEV)]
    mu.grasp_step([dev(seeded(81, rows, cols))], gs, [G], MU, LR, 0.0, "standard", M_out=Mt)
    torch.cuda.synchronize()
    g_stored = syn.to_f64(G).astype(np.float32)  # the bf16 values the kernel read
    _, st1, _, M1, _ = go.grasp_step(seeded(81, rows, cols).astype(np.float64), go.new_state(rows, cols, 0),
                                     g_stored, MU, LR)
    assert np.array_equal(host(Mt[0]), M1.astype(np.float32))
    assert np.array_equal(go.unpack_nibbles(host(gs.res_codes[0]), cols), st1["res_codes"])
    assert np.array_equal(host(gs.res_row_scales[0]), st1["res_sr"])
