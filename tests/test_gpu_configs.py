"""GPU parity on the parity subsets of the workloads (synthetic stand-ins for
the pages' settings), through the C ABI:

* the LLaMA-130M-shaped set in full (48 x 768x768 and 36 x 768x2048, bf16
  state, G ~ N(0, 1e-6)), standard NS;
* layer 0 of the LLaMA-1.1B-shaped set (4 x 2048x2048 and 3 x 2048x5632,
  momentum U diag(i^-1/2) V^T with Haar U, V), standard and Gram NS;
* 3 experts of the 64-expert MoE set (6 x 7168x2048, iterated transposed, and
  3 x 2048x7168, 1 % of the gradient entries scaled by 50), Gram NS.

One muon_step per same-shape group, each matrix then compared with the fp64
oracle: the stored momentum bit for bit, O at relative Frobenius 2e-2 (16-bit
operands), and the weight update at the O tolerance.
"""
import numpy as np
import pytest
import torch

import matrix_orthogonalizing_optimizer_step_amd as mu
from oracle import muon_oracle as orc
from synth import inputs as syn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MU, LR = 0.95, 0.02
TOL = 2e-2


def check_group(wl, gi, count, variant):
    Ws, Ms, Gs = syn.group_inputs(wl, gi, count=count)
    W = [w.to(DEV) for w in Ws]
    M = [m.to(DEV) for m in Ms]
    O = [torch.empty(w.shape, dtype=torch.float32, device=DEV) for w in Ws]
    mu.muon_step(W, M, [g.to(DEV) for g in Gs], MU, LR, 0.0, variant, None, O_out=O)
    torch.cuda.synchronize()
    mu32, lr32 = float(np.float32(MU)), float(np.float32(LR))
    worst = 0.0
    for i in range(len(Ws)):
        W0 = syn.to_f64(Ws[i])
        Wr, Mr, Or = orc.muon_step(W0, syn.to_f64(Ms[i]), syn.to_f64(Gs[i]), mu32, lr32, 0.0, variant,
                                   state_dtype=wl.state_dtype, w_dtype="f64")
        assert np.array_equal(syn.to_f64(M[i]), Mr), (wl.key, gi, i)
        err = orc.relative_frobenius(syn.to_f64(O[i]), Or)
        assert err < TOL, (wl.key, gi, i, err)
        dW = syn.to_f64(W[i]) - W0
        assert orc.relative_frobenius(dW, Wr - W0) < TOL + 1e-4, (wl.key, gi, i)
        worst = max(worst, err)
    print(f"{wl.key} group {gi} ({len(Ws)} x {Ws[0].shape[0]}x{Ws[0].shape[1]}) {variant}: max relF {worst:.2e}")


@pytest.mark.parametrize("gi", [0, 1], ids=["attn-768x768", "mlp-768x2048"])
def test_llama130m_all_matrices_standard(gi):
    check_group(syn.WORKLOADS["llama-130m"], gi, None, "standard")


@pytest.mark.parametrize("variant", ["standard", "gram"])
@pytest.mark.parametrize("gi,count", [(0, 4), (1, 3)], ids=["attn-2048x2048", "mlp-2048x5632"])
def test_llama1b_layer0(gi, count, variant):
    check_group(syn.WORKLOADS["llama-1.1b"], gi, count, variant)


@pytest.mark.parametrize("gi,count", [(0, 6), (1, 3)], ids=["up_gate-7168x2048", "down-2048x7168"])
def test_moe_three_experts_gram(gi, count):
    check_group(syn.WORKLOADS["moe-64x"], gi, count, "gram")


@pytest.mark.parametrize("wkey,gi,count", [("moe-64x", 0, 2), ("llama-130m", 0, 4)],
                         ids=["moe-up_gate-7168x2048", "llama130m-attn-768x768"])
def test_low_bit_state_first_step(wkey, gi, count):
    """The low-bit momentum state on a workload's own shapes and gradients
    (k = rank / 16), from the start state (zero residual and P, a seeded
    Gaussian R): M_t = G bit for bit, then the new state against the oracle's
    (codes off by one only at near-ties) and O at the 16-bit tolerance, one
    batched call per group."""
    from oracle import grasp_oracle as go
    from tests.test_gpu_grasp import compare_state
    wl = syn.WORKLOADS[wkey]
    Ws, _, Gs = syn.group_inputs(wl, gi, count=count)
    rows, cols = Ws[0].shape
    k = min(rows, cols) // 16
    R0 = [syn.random_matrix(500 + i, cols, k) for i in range(count)]
    gs = mu.GraspState(count, rows, cols, k, DEV, R_init=[r.to(DEV) for r in R0])
    W = [w.to(DEV) for w in Ws]
    O = [torch.empty(rows, cols, dtype=torch.float32, device=DEV) for _ in Ws]
    Mt = [torch.empty(rows, cols, dtype=torch.float32, device=DEV) for _ in Ws]
    mu.grasp_step(W, gs, [g.to(DEV) for g in Gs], MU, LR, 0.0, "gram", O_out=O, M_out=Mt)
    torch.cuda.synchronize()
    mu32, lr32 = float(np.float32(MU)), float(np.float32(LR))
    for i in range(count):
        st = go.new_state(rows, cols, k, R_init=syn.to_f64(R0[i]).astype(np.float32))
        G = syn.to_f64(Gs[i]).astype(np.float32)
        W1, st1, O1, M1, det = go.grasp_step(syn.to_f64(Ws[i]), st, G, mu32, lr32, 0.0, "gram")
        assert np.array_equal(syn.to_f64(Mt[i]), M1), i
        one = mu.GraspState(1, rows, cols, 0, DEV)
        one.k = k
        for name in ("res_codes", "res_row_scales", "res_col_scales", "P_codes", "P_scales", "R_codes", "R_scales"):
            setattr(one, name, [getattr(gs, name)[i]])
        compare_state(one, st1, det, rows, cols, k, M_ref=M1)
        assert orc.relative_frobenius(syn.to_f64(O[i]), O1) < TOL, i
