"""Seeded synthetic inputs for the Muon step (no method arithmetic here).

Both the HIP path's tests/benchmark and the oracle read their inputs from
this module; it only draws random numbers and shapes them.  Every tensor is
drawn from numpy's PCG64 seeded with SeedSequence((2026, config, matrix,
tensor)) in float32 and then stored in its dtype (bfloat16 values are made
with torch's round-to-nearest-even conversion), so both sides see the same
exact values.

Workloads stand in for the pages' settings (LLaMA pretraining and Qwen2.5-7B
fine-tuning in the low-bit Muon notes, the Kimi-K2-scale MoE in the Gram
Newton-Schulz notes).  No dataset or checkpoint is used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

TENSOR_W, TENSOR_M, TENSOR_G, TENSOR_U, TENSOR_V, TENSOR_MASK = range(6)

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Group:
    """A batch of same-shape matrices inside a workload."""
    name: str
    rows: int
    cols: int
    count: int


@dataclass(frozen=True)
class Workload:
    key: str
    cid: int            # the config number used in the seeds
    groups: tuple
    w_dtype: str
    state_dtype: str
    grad_std: float     # standard deviation of the gradient entries
    prev_momentum: str  # "zero", "gaussian" or "spectrum"
    outliers: float     # fraction of gradient entries scaled by 50 (0 = none)
    description: str

    @property
    def matrices(self):
        return sum(g.count for g in self.groups)

    @property
    def elements(self):
        return sum(g.count * g.rows * g.cols for g in self.groups)


WORKLOADS = {
    "single-256x512": Workload(
        "single-256x512", 1, (Group("w", 256, 512, 1),), "f32", "f32", 1.0, "gaussian", 0.0,
        "one 256x512 fp32 weight; W, M and G i.i.d. N(0,1); mu=0.95, lr=0.02"),
    "llama-130m": Workload(
        "llama-130m", 2,
        (Group("attn", 768, 768, 48), Group("mlp", 768, 2048, 36)),
        "f32", "bf16", 1e-3, "zero", 0.0,
        "12 layers x (4 attention 768x768 + 3 MLP 768x2048); bf16 state, G ~ N(0, 1e-6)"),
    "llama-1.1b": Workload(
        "llama-1.1b", 3,
        (Group("attn", 2048, 2048, 88), Group("mlp", 2048, 5632, 66)),
        "f32", "bf16", 0.0, "spectrum", 0.0,
        "22 layers x (4 of 2048x2048 + 3 of 2048x5632); momentum with spectrum i^-1/2"),
    "qwen2.5-7b": Workload(
        "qwen2.5-7b", 4,
        (Group("qo", 3584, 3584, 2), Group("kv", 3584, 512, 2), Group("mlp", 3584, 18944, 3)),
        "f32", "bf16", 1e-3, "zero", 0.0,
        "one layer: q,o 3584x3584; k,v 3584x512; gate,up,down 3584x18944"),
    "moe-64x": Workload(
        "moe-64x", 5,
        (Group("up_gate", 7168, 2048, 128), Group("down", 2048, 7168, 64)),
        "f32", "bf16", 1e-3, "zero", 0.01,
        "64 experts x (up, gate 7168x2048; down 2048x7168); 1% gradient outliers x50"),
}


def _rng(cid, matrix_id, tensor_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((2026, cid, matrix_id, tensor_id))))


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(_TORCH_DTYPES[dtype])


def gaussian(cid, matrix_id, tensor_id, rows, cols, std=1.0, dtype="f32"):
    """i.i.d. N(0, std^2) entries, stored in ``dtype``."""
    a = _rng(cid, matrix_id, tensor_id).standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return _store(a, dtype)


def haar_orthogonal(cid, matrix_id, tensor_id, n, k):
    """n x k matrix with orthonormal columns from the QR factorisation of a
    Gaussian matrix, signs fixed so the distribution is Haar."""
    g = _rng(cid, matrix_id, tensor_id).standard_normal((n, k))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def spectrum_matrix(cid, matrix_id, rows, cols, dtype="bf16"):
    """U diag(i^-1/2) V^T with Haar U, V (singular values 1, 1/sqrt 2, ...)."""
    k = min(rows, cols)
    U = haar_orthogonal(cid, matrix_id, TENSOR_U, rows, k)
    V = haar_orthogonal(cid, matrix_id, TENSOR_V, cols, k)
    s = np.arange(1, k + 1, dtype=np.float64) ** -0.5
    return _store(((U * s[None, :]) @ V.T).astype(np.float32), dtype)


def with_outliers(cid, matrix_id, G: torch.Tensor, frac: float, factor: float = 50.0):
    """Scale a seeded Bernoulli(frac) subset of the entries by ``factor``."""
    if frac <= 0:
        return G
    mask = _rng(cid, matrix_id, TENSOR_MASK).random(tuple(G.shape)) < frac
    g = G.to(torch.float32).numpy().copy()
    g[mask] *= np.float32(factor)
    return _store(g, {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[G.dtype])


def matrix_inputs(wl: Workload, matrix_id: int, rows: int, cols: int, step: int = 0):
    """(W, M_prev, G) for one matrix of a workload as CPU tensors in their
    dtypes.  ``step`` > 0 draws a fresh gradient for a later step (its seed
    tensor id is offset by 16 * step) and reuses W and M_prev."""
    cid = wl.cid
    W = gaussian(cid, matrix_id, TENSOR_W, rows, cols, 1.0, wl.w_dtype)
    if wl.prev_momentum == "gaussian":
        M = gaussian(cid, matrix_id, TENSOR_M, rows, cols, 1.0, wl.state_dtype)
    else:
        M = torch.zeros(rows, cols, dtype=_TORCH_DTYPES[wl.state_dtype])
    gid = TENSOR_G + 16 * step
    if wl.prev_momentum == "spectrum" and step == 0:
        G = spectrum_matrix(cid, matrix_id, rows, cols, wl.state_dtype)
    else:
        std = wl.grad_std if wl.grad_std > 0 else 1e-3
        G = gaussian(cid, matrix_id, gid, rows, cols, std, wl.state_dtype)
        G = with_outliers(cid, matrix_id * 1000 + step, G, wl.outliers)
    return W, M, G


def group_inputs(wl: Workload, group_index: int, count: int | None = None, step: int = 0):
    """Lists (W, M, G) for the first ``count`` matrices of one group."""
    g = wl.groups[group_index]
    base = sum(x.count for x in wl.groups[:group_index])
    count = g.count if count is None else min(count, g.count)
    Ws, Ms, Gs = [], [], []
    for i in range(count):
        W, M, G = matrix_inputs(wl, base + i, g.rows, g.cols, step)
        Ws.append(W)
        Ms.append(M)
        Gs.append(G)
    return Ws, Ms, Gs


def random_matrix(seed: int, rows: int, cols: int, std: float = 1.0, dtype: str = "f32"):
    """A free-standing seeded Gaussian matrix for unit tests."""
    return gaussian(9000 + seed, 0, 0, rows, cols, std, dtype)


def dyadic_matrix(seed: int, n: int, m: int, dtype: str = "bf16"):
    """An n x m matrix (n a power of two, n <= m) whose entries all come from
    one seeded Gaussian vector g of length n (stored in ``dtype``): the n x n
    block D[r][c] = g[r XOR c] sits in n columns chosen by a seeded
    permutation, each with a seeded sign; the other m - n columns are zero.
    Returns (matrix as a CPU tensor, g, the column of D for every output
    column or -1, the column signs).  Only random draws and index shuffling
    happen here."""
    if n & (n - 1) or n > m:
        raise ValueError("n must be a power of two and at most m")
    r = _rng(9700 + seed, n, m)
    g = r.standard_normal(n).astype(np.float32)
    g = _store(g[None, :], dtype).to(torch.float64).numpy()[0]
    perm = r.permutation(m)
    src = np.full(m, -1, dtype=np.int64)
    src[perm[:n]] = np.arange(n)
    signs = np.where(r.random(m) < 0.5, -1.0, 1.0)
    idx = np.arange(n, dtype=np.int32)
    D = g[np.bitwise_xor.outer(idx, idx)].astype(np.float32)
    out = np.zeros((n, m), dtype=np.float32)
    cols = perm[:n]
    out[:, cols] = D * signs[cols][None, :].astype(np.float32)
    return _store(out, dtype), g, src, signs


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU or device tensor's stored values."""
    return t.detach().to("cpu", torch.float64).numpy()


def random_codes(seed: int, shape, levels: int) -> np.ndarray:
    """Uniform integers in [-levels, levels] (int8): an arbitrary stored code."""
    r = _rng(9500 + seed, 0, 0)
    return r.integers(-levels, levels + 1, size=shape).astype(np.int8)


def random_scales(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Positive float32 values exp(N(0, 1/4)) * scale: arbitrary stored scales."""
    r = _rng(9600 + seed, 0, 0)
    return (np.exp(0.5 * r.standard_normal(shape)) * scale).astype(np.float32)
