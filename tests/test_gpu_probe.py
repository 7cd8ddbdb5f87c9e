"""The matrix-core rate probe bench.py reports next to the published peak (needs an
MI355X): its measured rate must be positive and cannot exceed the chip's published
dense bf16 peak by more than clock noise."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_mfma_probe_rate_is_plausible():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    print("[probe] 256 workgroups x 2000 rounds", flush=True)
    rate = bench.mfma_probe_tflops(blocks=256, iters=2000)
    print(f"[probe] {rate:.1f} TFLOP/s", flush=True)
    assert 100.0 < rate <= 1.05 * bench.MFMA_PEAK_BF16_TFLOPS
