"""ctypes binding of ``libmuon.so`` (the C ABI in include/muon.h).

Argument marshalling only: PyTorch supplies device memory and the stream;
every step of the computation runs in the library's HIP kernels.  The
functions keep the C names: ``ns_orthogonalize``, ``gram_ns_orthogonalize``
and ``muon_step`` take lists of same-shape device tensors (one per matrix of
the batch).  There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from collections import OrderedDict
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MUON_LIBRARY selects another build of the library (e.g. for A/B timing)
LIB_PATH = os.environ.get("MUON_LIBRARY") or os.path.join(_HERE, "libmuon.so")

F32, BF16, F16 = 0, 1, 2
STANDARD, GRAM = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_DT_NAMES = {"f32": F32, "bf16": BF16, "f16": F16}
_VARIANTS = {"standard": STANDARD, "gram": GRAM}


class MuonError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"muon status {status}: {msg}")
        self.status = status


class TraceRecord(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 40), ("role", ctypes.c_char * 24), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double), ("ms", ctypes.c_float)]


class _Config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("coeffs", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("restart_mask", ctypes.c_uint32), ("compute", ctypes.c_int), ("shift", ctypes.c_int32)]


class _GraspState(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("res_codes", "res_row_scales", "res_col_scales", "P_codes", "P_scales", "R_codes", "R_scales")]


_lib = None


def load_library():
    """Load libmuon.so once; raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m matrix_orthogonalizing_optimizer_step_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    cfgp = ctypes.POINTER(_Config)
    lib.muon_ns_config_init.argtypes = [cfgp, i32]
    lib.muon_ns_config_init.restype = None
    lib.muon_workspace_size.argtypes = [i32, i32, i32, i32, cfgp]
    lib.muon_workspace_size.restype = sz
    sig = [i32, i32, i32, vp, i32, vp, i32, cfgp, vp, sz, vp]
    for name in ("ns_orthogonalize", "gram_ns_orthogonalize"):
        f = getattr(lib, name)
        f.argtypes = sig
        f.restype = i32
    lib.muon_step.argtypes = [i32, i32, i32, vp, i32, vp, vp, i32, ctypes.c_float, ctypes.c_float,
                              ctypes.c_float, ctypes.c_float, i32, cfgp, vp, i32, vp, sz, vp]
    lib.muon_step.restype = i32
    lib.muon_step_fixed_scratch.argtypes = [i32, i32, i32, vp, i32, vp, vp, i32, ctypes.c_float, ctypes.c_float,
                                            ctypes.c_float, ctypes.c_float, i32, cfgp, vp, i32, vp]
    lib.muon_step_fixed_scratch.restype = i32
    lib.muon_ns_flops.argtypes = [i32, i32, i32, cfgp, i32]
    lib.muon_ns_flops.restype = ctypes.c_double
    lib.muon_status_string.argtypes = [i32]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_trace_enable.argtypes = [i32]
    lib.muon_trace_enable.restype = i32
    lib.muon_trace_collect.argtypes = [ctypes.POINTER(TraceRecord), i32]
    lib.muon_trace_collect.restype = i32
    lib.muon_mfma_ceiling.argtypes = [i32, i32, i32, vp, vp]
    lib.muon_mfma_ceiling.restype = i32
    lib.muon_abi_version.argtypes = []
    lib.muon_abi_version.restype = i32
    lib.muon_quintic_schedule.argtypes = [i32, ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_double)]
    lib.muon_quintic_schedule.restype = i32
    lib.muon_grasp_workspace_size.argtypes = [i32, i32, i32, i32, i32, cfgp]
    lib.muon_grasp_workspace_size.restype = sz
    lib.muon_grasp_step.argtypes = [i32, i32, i32, i32, vp, i32, ctypes.POINTER(_GraspState), vp, i32,
                                    ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, i32, cfgp,
                                    vp, i32, vp, vp, sz, vp, vp]
    lib.muon_grasp_step.restype = i32
    for name in ("muon_grid_quantize", "muon_grid_dequantize"):
        getattr(lib, name).argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        getattr(lib, name).restype = i32
    for name in ("muon_group8_quantize", "muon_group8_dequantize"):
        getattr(lib, name).argtypes = [i32, i32, i32, vp, vp, vp, vp]
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


@dataclass
class NSConfig:
    """Python view of muon_ns_config; None fields take the variant default."""
    T: int = 5
    coeffs: Optional[Sequence[Sequence[float]]] = None
    eps: float = 1e-7
    restart_mask: Optional[int] = None
    compute: Optional[str] = None  # "bf16", "f16" or "f32"
    shift: bool = True

    def to_c(self, variant: int):
        lib = load_library()
        c = _Config()
        lib.muon_ns_config_init(ctypes.byref(c), variant)
        c.T = int(self.T)
        c.eps = float(self.eps)
        if self.restart_mask is not None:
            c.restart_mask = int(self.restart_mask)
        if self.compute is not None:
            c.compute = _DT_NAMES[self.compute]
        c.shift = 1 if self.shift else 0
        keep = None
        if self.coeffs is not None:
            flat = [float(x) for row in self.coeffs for x in row]
            keep = (ctypes.c_float * len(flat))(*flat)
            c.coeffs = ctypes.cast(keep, ctypes.c_void_p)
        return c, keep


def _variant(v) -> int:
    return _VARIANTS[v] if isinstance(v, str) else int(v)


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise MuonError(status, lib.muon_status_string(status).decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _stream_obj(stream, device):
    """The torch stream object for None (current), a torch stream or a raw handle."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


class _PtrArray:
    """A cached pointer array: the device tensor, the stream its copy was
    enqueued on, and an event recorded after that copy."""
    __slots__ = ("arr", "stream", "ready")

    def __init__(self, arr, stream, ready):
        self.arr, self.stream, self.ready = arr, stream, ready


_ptr_cache: "OrderedDict[tuple, _PtrArray]" = OrderedDict()  # least recently used first
_ptr_pinned: dict = {}  # arrays a captured graph reads: kept for the life of the process
_PTR_CACHE_MAX = 256


def pointer_array(tensors: Sequence[torch.Tensor], stream=None) -> torch.Tensor:
    """A device array holding the data pointers of ``tensors``, for use on
    ``stream`` (None = the current stream).

    A new array is filled by an asynchronous copy from pinned host memory
    enqueued on ``stream``, so the host never waits for the device.  Arrays
    are cached by device and pointers (least recently used dropped past 256
    entries).  Using a cached array on another stream first waits, on the
    host, for the event after its copy (only if that copy has not finished,
    which is rare) and records the stream with the caching allocator, so a
    dropped array's memory is not reused while that stream may still read
    it.  Making an array is a copy, which a stream under graph capture does
    not take: call once with the same tensors before capturing.  An array used
    during a capture is kept for the life of the process, since the graph
    reads it at every replay."""
    ptrs = tuple(int(t.data_ptr()) for t in tensors)
    dev = tensors[0].device
    key = (str(dev), ptrs)
    if dev.type != "cuda":  # host tensors (argument checks without a device)
        ent = _ptr_cache.get(key)
        if ent is None:
            while len(_ptr_cache) >= _PTR_CACHE_MAX:
                _ptr_cache.popitem(last=False)
            ent = _ptr_cache[key] = _PtrArray(torch.tensor(ptrs, dtype=torch.int64), None, None)
        else:
            _ptr_cache.move_to_end(key)
        return ent.arr
    capturing = torch.cuda.is_current_stream_capturing()
    ent = _ptr_pinned.get(key)
    if ent is None:
        ent = _ptr_cache.get(key)
        if ent is None:
            if capturing:
                raise MuonError(1, "pointer array not cached for these tensors: under graph capture, "
                                   "call once with the same tensors before capturing")  # MUON_ERR_INVALID_ARG
            while len(_ptr_cache) >= _PTR_CACHE_MAX:
                _ptr_cache.popitem(last=False)  # its streams are recorded: freeing it is ordered after them
            s = _stream_obj(stream, dev)
            host = torch.tensor(ptrs, dtype=torch.int64).pin_memory()
            with torch.cuda.stream(s):
                arr = torch.empty(len(ptrs), dtype=torch.int64, device=dev)
                arr.copy_(host, non_blocking=True)
                ready = torch.cuda.Event()
                ready.record(s)
            ent = _ptr_cache[key] = _PtrArray(arr, s.cuda_stream, ready)
            return ent.arr
        _ptr_cache.move_to_end(key)
        if capturing:
            _ptr_pinned[key] = _ptr_cache.pop(key)
    if capturing:  # a capture starts with a device synchronisation: the copy has landed
        return ent.arr
    if _stream(stream) != ent.stream:
        if not ent.ready.query():
            ent.ready.synchronize()
        if key not in _ptr_pinned:
            ent.arr.record_stream(_stream_obj(stream, dev))
    return ent.arr


def _batch(tensors: Sequence[torch.Tensor], name: str):
    if len(tensors) == 0:
        raise ValueError(f"{name}: empty batch")
    t0 = tensors[0]
    if t0.dim() != 2:
        raise ValueError(f"{name}: matrices must be 2-D")
    for t in tensors:
        if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError(f"{name}: all matrices must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError(f"{name}: matrices must be contiguous")
        if t.device.type != "cuda":
            raise ValueError(f"{name}: matrices must be device tensors")
    return t0.shape[0], t0.shape[1], _DT[t0.dtype]


_ws_cache: dict = {}   # (device, stream handle) -> buffer
_ws_pinned: dict = {}  # buffers a captured graph uses: kept for the life of the process


def workspace_size(batch: int, rows: int, cols: int, variant="standard", cfg: Optional[NSConfig] = None) -> int:
    lib = load_library()
    v = _variant(variant)
    c, _keep = (cfg or NSConfig()).to_c(v)
    n = lib.muon_workspace_size(batch, rows, cols, v, ctypes.byref(c))
    if n == 0:
        raise MuonError(1, "invalid arguments for the workspace size")
    return int(n)


def workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    """A cached device byte buffer of at least ``nbytes`` (256-byte aligned)
    for calls on ``stream`` (None = the current stream).

    One buffer per (device, stream): calls on different streams never share
    scratch memory.  A buffer is allocated on its stream, so when a larger one
    replaces it the caching allocator reuses its memory only in that stream's
    order, after the calls that used it.  A buffer used during a graph
    capture is kept for the life of the process (the graph uses it at every
    replay) and never replaced: a larger need then gets a new buffer."""
    dev = torch.device(device)
    s = _stream_obj(stream, dev)
    key = (str(dev), s.cuda_stream)
    capturing = torch.cuda.is_current_stream_capturing()
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    if capturing:
        _ws_pinned[buf.data_ptr()] = buf
    return buf


def _orthogonalize(fname, variant, M, O, cfg, ws, stream):
    lib = load_library()
    rows, cols, mdt = _batch(M, "M")
    _, _, odt = _batch(O, "O")
    if tuple(O[0].shape) != (rows, cols) or len(O) != len(M):
        raise ValueError("O must match M")
    c, _keep = (cfg or NSConfig()).to_c(variant)
    need = lib.muon_workspace_size(len(M), rows, cols, variant, ctypes.byref(c))
    if ws is None:
        ws = workspace(need, M[0].device, stream)
    pm, po = pointer_array(M, stream), pointer_array(O, stream)
    st = getattr(lib, fname)(len(M), rows, cols, pm.data_ptr(), mdt, po.data_ptr(), odt, ctypes.byref(c),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st)
    return O


def ns_orthogonalize(M, O, cfg: Optional[NSConfig] = None, workspace=None, stream=None):
    """Standard Newton-Schulz of every matrix in ``M`` into ``O`` (lists of tensors)."""
    return _orthogonalize("ns_orthogonalize", STANDARD, M, O, cfg, workspace, stream)


def gram_ns_orthogonalize(M, O, cfg: Optional[NSConfig] = None, workspace=None, stream=None):
    """Gram Newton-Schulz of every matrix in ``M`` into ``O`` (lists of tensors)."""
    return _orthogonalize("gram_ns_orthogonalize", GRAM, M, O, cfg, workspace, stream)


def muon_step(W, M, G, mu: float, lr: float, weight_decay: float = 0.0, variant="standard",
              cfg: Optional[NSConfig] = None, O_out=None, workspace=None, stream=None,
              update_scale: float = 1.0):
    """One Muon step on lists of same-shape tensors; W and M are updated in place:
    W <- W - lr (update_scale O + weight_decay W)."""
    lib = load_library()
    v = _variant(variant)
    rows, cols, wdt = _batch(W, "W")
    r2, c2, sdt = _batch(M, "M")
    r3, c3, gdt = _batch(G, "G")
    if (r2, c2) != (rows, cols) or (r3, c3) != (rows, cols) or gdt != sdt:
        raise ValueError("W, M and G must share the shape; M and G the dtype")
    if not (len(W) == len(M) == len(G)):
        raise ValueError("W, M and G must have one tensor per matrix")
    c, _keep = (cfg or NSConfig()).to_c(v)
    need = lib.muon_workspace_size(len(W), rows, cols, v, ctypes.byref(c))
    if workspace is None:
        workspace = globals()["workspace"](need, W[0].device, stream)
    po, odt = None, F32
    if O_out is not None:
        _, _, odt = _batch(O_out, "O_out")
        po = pointer_array(O_out, stream)
    pw, pm, pg = pointer_array(W, stream), pointer_array(M, stream), pointer_array(G, stream)
    st = lib.muon_step(len(W), rows, cols, pw.data_ptr(), wdt, pm.data_ptr(), pg.data_ptr(), sdt,
                       float(mu), float(lr), float(weight_decay), float(update_scale), v, ctypes.byref(c),
                       po.data_ptr() if po is not None else None, odt,
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st)


FIXED_SCRATCH_BYTES = 64 << 20  # MUON_FIXED_SCRATCH_BYTES


def muon_step_fixed_scratch(W, M, G, mu: float, lr: float, weight_decay: float = 0.0, variant="standard",
                            cfg: Optional[NSConfig] = None, O_out=None, stream=None, update_scale: float = 1.0):
    """muon_step with the library's fixed device scratch instead of a
    workspace (for callers that cannot allocate; problems whose workspace
    exceeds FIXED_SCRATCH_BYTES are refused).  Calls that overlap on one
    device race on that scratch."""
    lib = load_library()
    v = _variant(variant)
    rows, cols, wdt = _batch(W, "W")
    r2, c2, sdt = _batch(M, "M")
    r3, c3, gdt = _batch(G, "G")
    if (r2, c2) != (rows, cols) or (r3, c3) != (rows, cols) or gdt != sdt:
        raise ValueError("W, M and G must share the shape; M and G the dtype")
    if not (len(W) == len(M) == len(G)):
        raise ValueError("W, M and G must have one tensor per matrix")
    c, _keep = (cfg or NSConfig()).to_c(v)
    po, odt = None, F32
    if O_out is not None:
        _, _, odt = _batch(O_out, "O_out")
        po = pointer_array(O_out, stream)
    pw, pm, pg = pointer_array(W, stream), pointer_array(M, stream), pointer_array(G, stream)
    st = lib.muon_step_fixed_scratch(len(W), rows, cols, pw.data_ptr(), wdt, pm.data_ptr(), pg.data_ptr(), sdt,
                                     float(mu), float(lr), float(weight_decay), float(update_scale), v,
                                     ctypes.byref(c), po.data_ptr() if po is not None else None, odt,
                                     _stream(stream))
    _check(st)


def ns_flops(rows: int, cols: int, variant="standard", cfg: Optional[NSConfig] = None,
             symmetric_aware: bool = True) -> float:
    """FLOPs of one orthogonalisation (see muon_ns_flops in include/muon.h)."""
    lib = load_library()
    v = _variant(variant)
    c, _keep = (cfg or NSConfig()).to_c(v)
    return float(lib.muon_ns_flops(rows, cols, v, ctypes.byref(c), 1 if symmetric_aware else 0))


def quintic_schedule(T: int = 5, ell: float = 1e-3, safety: float = 1.0):
    """Per-iteration minimax quintics (see muon_quintic_schedule in
    include/muon.h).  Returns (coeffs, bounds): T (a, b, c) tuples of fp32
    values, usable as NSConfig.coeffs, and the T + 1 intervals (l_t, u_t)."""
    lib = load_library()
    c = (ctypes.c_float * (3 * T))()
    b = (ctypes.c_double * (2 * T + 2))()
    _check(lib.muon_quintic_schedule(int(T), float(ell), float(safety), c, b))
    coeffs = [(c[3 * t], c[3 * t + 1], c[3 * t + 2]) for t in range(T)]
    bounds = [(b[2 * t], b[2 * t + 1]) for t in range(T + 1)]
    return coeffs, bounds


def abi_version() -> int:
    return int(load_library().muon_abi_version())


def trace_enable(on: bool = True) -> bool:
    """Turn the library's launch trace on or off (clears it); returns the old setting."""
    return bool(load_library().muon_trace_enable(1 if on else 0))


def mfma_ceiling(blocks: int, rounds: int, sink: torch.Tensor, dtype: str = "f16", stream=None):
    """Enqueue the register-only MFMA probe (muon_mfma_ceiling) of operand
    type ``dtype`` ("f16" or "bf16") on the stream; ``sink`` is a float32
    device tensor of at least blocks * 256 elements.  Returns the FLOPs the
    launch performs (time it with events)."""
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks * 256:
        raise ValueError("sink must be a float32 device tensor of at least blocks * 256 elements")
    codes = {"f16": F16, "bf16": BF16}
    if dtype not in codes:
        raise ValueError("dtype must be 'f16' or 'bf16'")
    _check(load_library().muon_mfma_ceiling(blocks, rounds, codes[dtype], ctypes.c_void_p(sink.data_ptr()),
                                            ctypes.c_void_p(_stream(stream))))
    return float(blocks) * 4 * 32 * rounds * 32768.0


def trace_collect():
    """Wait for the traced launches and return them as dicts (oldest first)."""
    lib = load_library()
    cap = 1 << 16
    buf = (TraceRecord * cap)()
    n = lib.muon_trace_collect(buf, cap)
    if n < 0:
        raise MuonError(4, "trace event query failed")
    if n > cap:
        raise MuonError(1, f"trace held {n} records, more than {cap}")
    return [dict(kernel=buf[i].kernel.decode(), role=buf[i].role.decode(), flops=buf[i].flops,
                 bytes=buf[i].bytes, ms=float(buf[i].ms)) for i in range(n)]


# --------------------------------------------------------------------------
# low-bit momentum state (muon_grasp_state and muon_grasp_step in include/muon.h)
# --------------------------------------------------------------------------
GRID = 128  # grid block edge and 8-bit group length


def _nb(x: int) -> int:
    return (x + GRID - 1) // GRID


def grid_quantize(X, stream=None):
    """4-bit grid code of fp32 matrices: returns (codes, row_scales, col_scales) lists."""
    lib = load_library()
    rows, cols, dt = _batch(X, "X")
    if dt != F32:
        raise ValueError("X must be float32")
    dev = X[0].device
    codes = [torch.empty(rows, (cols + 1) // 2, dtype=torch.uint8, device=dev) for _ in X]
    sr = [torch.empty(rows, _nb(cols), dtype=torch.float32, device=dev) for _ in X]
    sc = [torch.empty(_nb(rows), cols, dtype=torch.float32, device=dev) for _ in X]
    _check(lib.muon_grid_quantize(len(X), rows, cols, pointer_array(X, stream).data_ptr(), pointer_array(codes, stream).data_ptr(),
                                  pointer_array(sr, stream).data_ptr(), pointer_array(sc, stream).data_ptr(), _stream(stream)))
    return codes, sr, sc


def grid_dequantize(codes, row_scales, col_scales, cols: int, stream=None):
    """fp32 values q m / 7 of 4-bit grid codes (rows x cols each)."""
    lib = load_library()
    rows = codes[0].shape[0]
    dev = codes[0].device
    Y = [torch.empty(rows, cols, dtype=torch.float32, device=dev) for _ in codes]
    _check(lib.muon_grid_dequantize(len(codes), rows, cols, pointer_array(codes, stream).data_ptr(),
                                    pointer_array(row_scales, stream).data_ptr(), pointer_array(col_scales, stream).data_ptr(),
                                    pointer_array(Y, stream).data_ptr(), _stream(stream)))
    return Y


def group8_quantize(X, stream=None):
    """8-bit group code (groups of 128 along rows) of fp32 matrices: (codes, scales)."""
    lib = load_library()
    rows, k, dt = _batch(X, "X")
    if dt != F32:
        raise ValueError("X must be float32")
    dev = X[0].device
    codes = [torch.empty(rows, k, dtype=torch.int8, device=dev) for _ in X]
    scales = [torch.empty(rows, _nb(k), dtype=torch.float32, device=dev) for _ in X]
    _check(lib.muon_group8_quantize(len(X), rows, k, pointer_array(X, stream).data_ptr(), pointer_array(codes, stream).data_ptr(),
                                    pointer_array(scales, stream).data_ptr(), _stream(stream)))
    return codes, scales


def group8_dequantize(codes, scales, stream=None):
    lib = load_library()
    rows, k = codes[0].shape
    Y = [torch.empty(rows, k, dtype=torch.float32, device=codes[0].device) for _ in codes]
    _check(lib.muon_group8_dequantize(len(codes), rows, k, pointer_array(codes, stream).data_ptr(),
                                      pointer_array(scales, stream).data_ptr(), pointer_array(Y, stream).data_ptr(), _stream(stream)))
    return Y


class GraspState:
    """Device buffers of the low-bit momentum state of ``batch`` rows x cols
    matrices with subspace rank k (layout of muon_grasp_state).  The residual
    and P start at zero; R starts as the 8-bit code of ``R_init`` (a list of
    fp32 cols x k tensors), required when k > 0."""

    def __init__(self, batch: int, rows: int, cols: int, k: int, device, R_init=None):
        z = lambda *shape, dt: torch.zeros(*shape, dtype=dt, device=device)  # noqa: E731
        self.rows, self.cols, self.k, self.batch = rows, cols, k, batch
        self.res_codes = [z(rows, (cols + 1) // 2, dt=torch.uint8) for _ in range(batch)]
        self.res_row_scales = [z(rows, _nb(cols), dt=torch.float32) for _ in range(batch)]
        self.res_col_scales = [z(_nb(rows), cols, dt=torch.float32) for _ in range(batch)]
        self.P_codes = self.P_scales = self.R_codes = self.R_scales = None
        if k > 0:
            if R_init is None or len(R_init) != batch:
                raise ValueError("k > 0 needs one cols x k start matrix R_init per matrix")
            self.P_codes = [z(rows, k, dt=torch.int8) for _ in range(batch)]
            self.P_scales = [z(rows, _nb(k), dt=torch.float32) for _ in range(batch)]
            self.R_codes, self.R_scales = group8_quantize([r.to(device, torch.float32).contiguous() for r in R_init])

    def c_struct(self, stream=None):
        st = _GraspState()
        keep = []
        for name in ("res_codes", "res_row_scales", "res_col_scales", "P_codes", "P_scales", "R_codes", "R_scales"):
            lst = getattr(self, name)
            if lst is not None:
                arr = pointer_array(lst, stream)
                keep.append(arr)
                setattr(st, name, arr.data_ptr())
        return st, keep


def grasp_workspace_size(batch: int, rows: int, cols: int, k: int, variant="standard",
                         cfg: Optional[NSConfig] = None) -> int:
    lib = load_library()
    v = _variant(variant)
    c, _keep = (cfg or NSConfig()).to_c(v)
    n = lib.muon_grasp_workspace_size(batch, rows, cols, k, v, ctypes.byref(c))
    if n == 0:
        raise MuonError(1, "invalid arguments for the workspace size")
    return int(n)


def grasp_step(W, state: GraspState, G, mu: float, lr: float, weight_decay: float = 0.0, variant="standard",
               cfg: Optional[NSConfig] = None, O_out=None, M_out=None, workspace=None, stream=None,
               update_scale: float = 1.0, aux_stream=None):
    """One Muon step whose momentum lives in ``state`` (updated in place with W).
    ``aux_stream``: a second stream on which the state update runs beside
    Newton-Schulz (joined back into ``stream`` at the end of the call)."""
    lib = load_library()
    v = _variant(variant)
    rows, cols, wdt = _batch(W, "W")
    r3, c3, gdt = _batch(G, "G")
    if (r3, c3) != (rows, cols) or (state.rows, state.cols) != (rows, cols) or not (len(W) == len(G) == state.batch):
        raise ValueError("W, G and the state must match")
    c, _keep = (cfg or NSConfig()).to_c(v)
    need = lib.muon_grasp_workspace_size(len(W), rows, cols, state.k, v, ctypes.byref(c))
    if need == 0:
        raise MuonError(1, "invalid arguments for the workspace size")
    if workspace is None:
        workspace = globals()["workspace"](need, W[0].device, stream)
    po, odt = None, F32
    if O_out is not None:
        _, _, odt = _batch(O_out, "O_out")
        po = pointer_array(O_out, stream)
    pm = pointer_array(M_out, stream) if M_out is not None else None
    st, _keep_st = state.c_struct(stream)
    st_ = lib.muon_grasp_step(len(W), rows, cols, state.k, pointer_array(W, stream).data_ptr(), wdt,
                              ctypes.byref(st), pointer_array(G, stream).data_ptr(), gdt, float(mu), float(lr), float(weight_decay),
                              float(update_scale), v, ctypes.byref(c),
                              po.data_ptr() if po is not None else None, odt,
                              pm.data_ptr() if pm is not None else None,
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream),
                              _stream(aux_stream) if aux_stream is not None else None)
    _check(st_)
