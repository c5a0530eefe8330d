"""muon_step_fixed_scratch (the step for callers that cannot allocate) against
muon_step with a workspace: the same kernels on the same inputs, so W, M and
O agree bit for bit.  Two calls in a row, the second on a smaller problem
(the scratch keeps the first call's contents), then a problem over the
scratch's size is refused before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import matrix_orthogonalizing_optimizer_step_amd as mu
from matrix_orthogonalizing_optimizer_step_amd import binding as bd
from oracle import muon_oracle as orc
from synth import inputs as syn

DEV = "cuda:0"


def test_fixed_scratch_refusals_need_no_device():
    """Host-side checks of the entry point (bogus pointers are never used)."""
    lib = mu.load_library()

    def call(batch=1, rows=4, cols=4, W=1, M=2, G=3, v=0, cfg=None):
        return lib.muon_step_fixed_scratch(batch, rows, cols, W, 0, M, G, 1, 0.9, 0.1, 0.0, 1.0, v, cfg, None, 0,
                                           None)

    assert call(W=None) == 1 and call(M=1) == 1 and call(batch=0) == 1
    c, _ = bd.NSConfig(compute="bf16").to_c(bd.GRAM)
    assert call(v=1, cfg=ctypes.byref(c)) == 2
    # 4096 x 4096 needs far more than the fixed scratch
    assert mu.workspace_size(1, 4096, 4096) > bd.FIXED_SCRATCH_BYTES
    assert call(rows=4096, cols=4096) == 3


def inputs(shape, batch, seed):
    r, c = shape
    Ws = [syn.random_matrix(seed + 3 * i, r, c) for i in range(batch)]
    Ms = [syn.random_matrix(seed + 3 * i + 1, r, c, std=1e-3, dtype="bf16") for i in range(batch)]
    Gs = [syn.random_matrix(seed + 3 * i + 2, r, c, std=1e-3, dtype="bf16") for i in range(batch)]
    return Ws, Ms, Gs


def run(fn, Ws, Ms, Gs, variant, **kw):
    W = [w.to(DEV) for w in Ws]
    M = [m.to(DEV) for m in Ms]
    G = [g.to(DEV) for g in Gs]
    O = [torch.empty(w.shape, dtype=torch.float32, device=DEV) for w in Ws]
    fn(W, M, G, 0.95, 0.02, 0.01, variant, None, O_out=O, **kw)
    torch.cuda.synchronize()
    return [t.cpu() for t in W], [t.cpu() for t in M], [t.cpu() for t in O]


@pytest.mark.gpu
@pytest.mark.parametrize("variant", ["standard", "gram"])
def test_fixed_scratch_matches_workspace_step(variant):
    # first a batch of two 768 x 2048 (about 18 MB of scratch), then a smaller
    # 300 x 200 problem on the scratch the first call left behind
    for shape, batch, seed in (((768, 2048), 2, 100), ((300, 200), 1, 200)):
        print(f"fixed scratch {variant} {batch} x {shape}", flush=True)
        assert mu.workspace_size(batch, *shape, variant) <= bd.FIXED_SCRATCH_BYTES
        Ws, Ms, Gs = inputs(shape, batch, seed)
        ref = run(mu.muon_step, Ws, Ms, Gs, variant)
        got = run(mu.muon_step_fixed_scratch, Ws, Ms, Gs, variant)
        for a, b in zip(ref, got):
            for x, y in zip(a, b):
                assert torch.equal(x, y)
        # and the oracle, at the 16-bit bar
        mu32, lr32, wd32 = (float(np.float32(v)) for v in (0.95, 0.02, 0.01))
        Wr, Mr, Or = orc.muon_step(syn.to_f64(Ws[0]), syn.to_f64(Ms[0]), syn.to_f64(Gs[0]), mu32, lr32, wd32,
                                   variant, state_dtype="bf16", w_dtype="f64")
        assert np.array_equal(syn.to_f64(got[1][0]), Mr)
        assert orc.relative_frobenius(syn.to_f64(got[2][0]), Or) < 2e-2
