"""The register-only MFMA probe behind bench.py's practical ceiling: it runs
through the C ABI, writes every sink element, and its rate lies between a
plausible floor and the dense peak at the nominal clock."""
import pytest
import torch

import matrix_orthogonalizing_optimizer_step_amd as mu

PEAK_16BIT_TFLOPS = 2516.6


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mfma_ceiling_probe_runs_and_is_below_the_dense_peak(dtype):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    mu.mfma_ceiling(blocks, 200, sink, dtype)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = mu.mfma_ceiling(blocks, 2000, sink, dtype)
    e1.record()
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) / 1e3) / 1e12
    print(f"register-only {dtype} MFMA rate {tflops:.0f} TFLOP/s", flush=True)
    assert bool(torch.isfinite(sink).all())
    assert 300.0 < tflops < 1.05 * PEAK_16BIT_TFLOPS
    with pytest.raises(ValueError):
        mu.mfma_ceiling(blocks, 10, sink[:100], dtype)
    with pytest.raises(ValueError):
        mu.mfma_ceiling(blocks, 10, sink, "f32")
