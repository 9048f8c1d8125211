"""The clock probe used to price kernels at the clock the chip runs at."""
import pytest

pytestmark = pytest.mark.gpu


def test_clock_probe_is_plausible():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dit_joint_self_amd as dj
    assert dj.dit_wall_clock_khz() > 0
    ghz, tflops = dj.dit_clock_probe(blocks=512, iters=2000)
    print(f"[clock probe] {ghz:.3f} GHz, {tflops:.0f} TFLOP/s", flush=True)
    assert 0.5 < ghz < 3.0
    # the probe's MFMA rate cannot exceed the dense bf16 rate at the measured clock
    assert 0 < tflops <= 256 * 4096 * ghz * 1e9 / 1e12 * 1.02
