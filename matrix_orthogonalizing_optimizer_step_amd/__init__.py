"""MI355X-native Muon optimizer step: momentum, standard or Gram Newton-Schulz
orthogonalisation and the weight update, in hand-written HIP kernels for
gfx950 behind the C ABI of include/muon.h.  This package is the thin ctypes
binding (``binding``) and the build script (``_build``)."""
from .binding import (  # noqa: F401
    BF16, F16, F32, GRAM, STANDARD, GraspState, MuonError, NSConfig, abi_version, grasp_step, grasp_workspace_size,
    gram_ns_orthogonalize, grid_dequantize, grid_quantize, group8_dequantize, group8_quantize, load_library,
    mfma_ceiling, muon_step, muon_step_fixed_scratch, ns_flops, ns_orthogonalize, pointer_array, quintic_schedule,
    trace_collect, trace_enable, workspace,
    workspace_size,
)
