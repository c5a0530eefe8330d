"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/muon.h declares, validates arguments before touching the
device, and its FLOP helper agrees with the oracle's counted products."""
import ctypes
import os
import re

import pytest

import matrix_orthogonalizing_optimizer_step_amd as mu
from matrix_orthogonalizing_optimizer_step_amd import binding as bd
from oracle import muon_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "muon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_library_exports_every_declared_function():
    lib = mu.load_library()
    names = header_functions()
    assert {"ns_orthogonalize", "gram_ns_orthogonalize", "muon_step", "muon_workspace_size"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert mu.abi_version() == 6


def test_status_strings():
    lib = mu.load_library()
    for s in range(5):
        assert lib.muon_status_string(s)
    assert lib.muon_status_string(99) == b"unknown status"


def test_default_config():
    c, _ = bd.NSConfig().to_c(bd.STANDARD)
    assert (c.T, c.restart_mask, c.compute, c.shift) == (5, 0, bd.BF16, 1)
    assert abs(c.eps - 1e-7) < 1e-12
    c, _ = bd.NSConfig().to_c(bd.GRAM)
    assert (c.restart_mask, c.compute) == (2, bd.F16)


@pytest.mark.parametrize("rows,cols", [(8, 8), (8, 32), (32, 8), (6, 18), (4, 32), (5, 7)])
@pytest.mark.parametrize("variant,restarts", [("standard", ()), ("gram", ()), ("gram", (2,)),
                                              ("gram", (1, 2, 3, 4)), ("gram", (1, 3))])
def test_flop_helper_matches_oracle_count(rows, cols, variant, restarts):
    mask = sum(1 << (t - 1) for t in restarts)
    cfg = bd.NSConfig(restart_mask=mask)
    d, s, _ = orc.counted_flops(rows, cols, variant, restarts=restarts)
    assert mu.ns_flops(rows, cols, variant, cfg, symmetric_aware=True) == s
    assert mu.ns_flops(rows, cols, variant, cfg, symmetric_aware=False) == d


def test_workspace_size_validation():
    assert mu.workspace_size(1, 256, 512) > 0
    assert mu.workspace_size(3, 512, 256, "gram") == mu.workspace_size(3, 256, 512, "gram")
    for args in [(0, 4, 4), (1, 0, 4), (1, 4, 0), (-1, 4, 4), (1, (1 << 20) + 1, 4)]:
        with pytest.raises(bd.MuonError):
            mu.workspace_size(*args)
    for cfg in [bd.NSConfig(T=0), bd.NSConfig(T=17), bd.NSConfig(eps=-1.0), bd.NSConfig(eps=float("nan")),
                bd.NSConfig(coeffs=[(1.0, float("inf"), 0.0)] * 5)]:
        with pytest.raises(bd.MuonError):
            mu.workspace_size(1, 4, 4, "standard", cfg)
    # a restart needs a later iteration: bit (t-1) with t >= T is rejected
    with pytest.raises(bd.MuonError):
        mu.workspace_size(1, 4, 4, "gram", bd.NSConfig(T=2, restart_mask=1 << 1))
    assert mu.workspace_size(1, 4, 4, "gram", bd.NSConfig(T=3, restart_mask=1 << 1)) > 0


def _call_orth(lib, batch=1, rows=4, cols=4, M=1, mdt=0, O=2, odt=0, cfg=None, ws=256, wsb=1 << 30):
    return lib.ns_orthogonalize(batch, rows, cols, M, mdt, O, odt, cfg, ws, wsb, None)


def test_invalid_calls_fail_before_any_device_work():
    """Each case is rejected by the host-side checks; no pointer is
    dereferenced, so bogus addresses are safe here."""
    lib = mu.load_library()
    ok_ws = mu.workspace_size(1, 4, 4)
    cases = [
        (dict(batch=0), 1), (dict(rows=0), 1), (dict(cols=-3), 1),
        (dict(M=None), 1), (dict(O=None), 1), (dict(O=1), 1),          # O aliases M
        (dict(mdt=7), 1), (dict(odt=2), 2),                           # f16 output unsupported
        (dict(ws=None), 3), (dict(wsb=ok_ws - 1), 3), (dict(ws=256 + 64), 3),
    ]
    for kw, code in cases:
        assert _call_orth(lib, **kw) == code, kw
    bad = bd._Config()
    lib.muon_ns_config_init(ctypes.byref(bad), 0)
    bad.T = 0
    assert _call_orth(lib, cfg=ctypes.byref(bad)) == 1
    bad.T = 5
    bad.compute = 9
    assert _call_orth(lib, cfg=ctypes.byref(bad)) == 1
    bad.compute = 1
    bad.shift = 3
    assert _call_orth(lib, cfg=ctypes.byref(bad)) == 1


def test_bf16_refused_for_gram_and_for_other_coefficient_tables():
    """bf16 operands are accepted for standard NS with the fixed quintic only:
    Gram NS computes in float16 (Gram NS notes, section 3.3) and other
    coefficient tables amplify bf16 rounding past the 16-bit tolerance.  The
    refusal is MUON_ERR_UNSUPPORTED, returned before any device work (bogus
    pointers are safe), and the workspace size is 0 for such a config."""
    lib = mu.load_library()

    def cfg_of(variant, compute, coeffs=None, T=5):
        c, keep = bd.NSConfig(T=T, compute=compute, coeffs=coeffs).to_c(variant)
        return c, keep

    quintic = [orc.QUINTIC] * 5
    cases = [(bd.GRAM, "bf16", None, 5, 2), (bd.GRAM, "bf16", quintic, 5, 2),
             (bd.STANDARD, "bf16", [(1.0, 0.0, 0.0)], 1, 2), (bd.STANDARD, "bf16", quintic[:4] + [(3.0, -3.2, 1.2)], 5, 2),
             (bd.STANDARD, "bf16", None, 5, 0), (bd.STANDARD, "bf16", quintic, 5, 0), (bd.STANDARD, "bf16", None, 3, 0),
             (bd.STANDARD, "f16", [(1.0, 0.0, 0.0)], 1, 0), (bd.GRAM, "f16", None, 5, 0), (bd.GRAM, "f32", None, 5, 0)]
    for variant, compute, coeffs, T, code in cases:
        c, keep = cfg_of(variant, compute, coeffs, T)
        if variant == bd.GRAM and T < 3:
            c.restart_mask = 0
        fn = lib.ns_orthogonalize if variant == bd.STANDARD else lib.gram_ns_orthogonalize
        ws = lib.muon_workspace_size(1, 4, 4, variant, ctypes.byref(c))
        if code == 0:
            assert ws > 0, (variant, compute, coeffs)
        else:
            assert ws == 0, (variant, compute, coeffs)
            assert fn(1, 4, 4, 1, 0, 2, 0, ctypes.byref(c), 256, 1 << 30, None) == code
            assert lib.muon_step(1, 4, 4, 1, 0, 2, 3, 1, 0.9, 0.1, 0.0, 1.0, variant, ctypes.byref(c), None, 0,
                                 256, 1 << 30, None) == code
            assert lib.muon_grasp_step(1, 8, 8, 0, 1, 0, ctypes.byref(bd._GraspState(*([16] * 7))), 2, 1, 0.9, 0.1,
                                       0.0, 1.0, variant, ctypes.byref(c), None, 0, None, 256, 1 << 30, None,
                                       None) == code
        del keep


def test_invalid_muon_step_calls():
    lib = mu.load_library()
    ws = mu.workspace_size(1, 4, 4)

    def call(W=1, wdt=0, M=2, G=3, sdt=1, mu_=0.9, lr=0.1, wd=0.0, s=1.0, v=0, O=None, odt=0, wsb=ws):
        return lib.muon_step(1, 4, 4, W, wdt, M, G, sdt, mu_, lr, wd, s, v, None, O, odt, 256, wsb, None)

    assert call(W=None) == 1
    assert call(M=1) == 1                 # aliasing
    assert call(O=3) == 1                 # O_out aliases G
    assert call(mu_=float("nan")) == 1
    assert call(lr=float("inf")) == 1
    assert call(s=float("nan")) == 1      # update scale must be finite
    assert call(wd=float("-inf")) == 1
    assert call(sdt=2) == 2               # f16 state unsupported
    assert call(wdt=2) == 2
    assert call(O=4, odt=2) == 2
    assert call(v=5) == 1
    assert call(wsb=ws - 1) == 3


def test_binding_rejects_bad_batches():
    import torch
    with pytest.raises(ValueError):
        bd._batch([], "M")
    with pytest.raises(ValueError):
        bd._batch([torch.zeros(3)], "M")
    with pytest.raises(ValueError):
        bd._batch([torch.zeros(3, 3), torch.zeros(3, 4)], "M")
    with pytest.raises(ValueError):
        bd._batch([torch.zeros(3, 3)], "M")  # not a device tensor


def test_invalid_grasp_calls():
    """Argument checks of the low-bit-state entry points (no device work)."""
    lib = mu.load_library()
    assert mu.grasp_workspace_size(1, 300, 200, 12) > mu.grasp_workspace_size(1, 300, 200, 0) > mu.workspace_size(1, 300, 200)
    for args in [(1, 8, 8, 9), (1, 8, 8, -1), (1, 2048, 2048, 1025), (0, 8, 8, 0)]:
        with pytest.raises(bd.MuonError):
            mu.grasp_workspace_size(*args)
    ws = mu.grasp_workspace_size(1, 8, 8, 2)
    full = bd._GraspState(*([16] * 7))

    def call(k=2, st=full, W=1, wdt=0, G=2, gdt=1, mu_=0.9, s=1.0, v=0, odt=0, O=None, wsb=ws, w=256):
        return lib.muon_grasp_step(1, 8, 8, k, W, wdt, ctypes.byref(st) if st is not None else None, G, gdt,
                                   mu_, 0.1, 0.0, s, v, None, O, odt, None, w, wsb, None, None)

    assert call(st=None) == 1
    assert call(st=bd._GraspState(16, 16, 16, None, None, None, None)) == 1   # k > 0 needs P and R
    assert call(k=9) == 1 and call(k=-1) == 1
    assert call(W=None) == 1 and call(G=None) == 1
    assert call(mu_=float("nan")) == 1 and call(s=float("inf")) == 1
    assert call(gdt=5) == 1 and call(v=3) == 1
    assert call(wdt=2) == 2 and call(O=4, odt=2) == 2
    assert call(wsb=ws - 1) == 3 and call(w=256 + 16) == 3
    assert call(G=1) == 1                                  # G aliases W
    assert lib.muon_grasp_step(8192, 8, 8, 0, 1, 0, ctypes.byref(full), 2, 1, 0.9, 0.1, 0.0, 1.0, 0, None, None, 0,
                               None, 256, 1 << 40, None, None) == 1   # batch over the limit
    assert lib.muon_grid_quantize(65536, 8, 8, 1, 2, 3, 4, None) == 1
    assert lib.muon_grid_quantize(0, 8, 8, 1, 2, 3, 4, None) == 1
    assert lib.muon_grid_quantize(1, 8, 8, None, 2, 3, 4, None) == 1
    assert lib.muon_grid_dequantize(1, 8, 0, 1, 2, 3, 4, None) == 1
    assert lib.muon_grid_dequantize(1, 8, 8, 1, 2, 3, None, None) == 1
    assert lib.muon_group8_quantize(1, 8, 0, 1, 2, 3, None) == 1
    assert lib.muon_group8_dequantize(1, 8, 8, 1, None, 3, None) == 1


def test_pointer_array_cache_evicts_least_recently_used():
    """The pointer-array cache drops the least recently used entry, so an array
    used just before a graph capture is still cached when the capture needs it."""
    import torch
    bd._ptr_cache.clear()
    keep = [torch.zeros(2)]
    first = bd.pointer_array(keep)
    others = [[torch.zeros(1)] for _ in range(bd._PTR_CACHE_MAX + 40)]
    for i, o in enumerate(others):
        bd.pointer_array(o)
        if i % 8 == 0:
            assert bd.pointer_array(keep) is first  # a hit moves it to the back
    assert len(bd._ptr_cache) <= bd._PTR_CACHE_MAX
    assert bd.pointer_array(keep) is first
    assert bd.pointer_array(keep).tolist() == [keep[0].data_ptr()]
    assert (str(keep[0].device), (others[0][0].data_ptr(),)) not in bd._ptr_cache
    bd._ptr_cache.clear()


def test_pointer_array_miss_under_capture_is_a_muon_error(monkeypatch):
    """Under graph capture an uncached pointer array is refused with the
    library's invalid-argument status (checked on the CPU by faking the
    capture state; no device work)."""
    import torch
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)

    class FakeDev:
        type = "cuda"

        def __str__(self):
            return "cuda:99"

    class FakeTensor:
        device = FakeDev()

        def data_ptr(self):
            return 0x1234500

    bd._ptr_cache.clear()
    with pytest.raises(bd.MuonError, match="before capturing") as e:
        bd.pointer_array([FakeTensor()])
    assert e.value.status == 1


def test_implicit_workspace_per_stream_and_pinned_under_capture(monkeypatch):
    """The binding's implicit workspace: one buffer per (device, stream),
    grown in place of the old one, and kept for good once a capture used it
    (checked on the CPU with stand-in streams and a faked capture state)."""
    import contextlib

    import torch

    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

    capturing = {"on": False}
    monkeypatch.setattr(torch.cuda, "stream", lambda s: contextlib.nullcontext())
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: capturing["on"])
    bd._ws_cache.clear()
    bd._ws_pinned.clear()
    s1, s2 = FakeStream(11), FakeStream(22)
    a = bd.workspace(1000, "cpu", s1)
    b = bd.workspace(1000, "cpu", s2)
    assert a.data_ptr() != b.data_ptr()               # streams never share scratch
    assert bd.workspace(500, "cpu", s1) is a          # reused while large enough
    c = bd.workspace(4000, "cpu", s1)                 # grown: a new buffer replaces the old one
    assert c is not a and c.numel() >= 4000 and bd.workspace(10, "cpu", s1) is c
    capturing["on"] = True
    d = bd.workspace(100, "cpu", s2)                  # used under capture: pinned
    assert d is b and bd._ws_pinned[d.data_ptr()] is d
    e = bd.workspace(8000, "cpu", s2)                 # a larger need under capture: new, also pinned
    assert e is not d and bd._ws_pinned[e.data_ptr()] is e and bd._ws_pinned[d.data_ptr()] is d
    capturing["on"] = False
    f = bd.workspace(16000, "cpu", s2)                # after the capture: replaced in the cache, pinned ones kept
    assert f is not e and bd._ws_pinned[e.data_ptr()] is e and f.data_ptr() not in bd._ws_pinned
    bd._ws_cache.clear()
    bd._ws_pinned.clear()


def test_mfma_ceiling_rejects_bad_arguments():
    """The ceiling probe checks its arguments before launching anything."""
    lib = mu.load_library()
    for blocks, rounds, dt, sink in ((0, 10, 2, 1024), (1 << 21, 10, 2, 1024), (4, 0, 1, 1024), (4, 10, 2, None),
                                     (4, 10, 0, 1024), (4, 10, 7, 1024)):
        assert lib.muon_mfma_ceiling(blocks, rounds, dt, sink, None) == 1  # MUON_ERR_INVALID_ARG
