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
