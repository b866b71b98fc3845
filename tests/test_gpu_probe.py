"""The device-wide barrier probe (a measurement entry point, not part of the
forward pass): every mode completes its rounds with every row read back as
written and no wait running out of polls."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_barrier_probe_rounds_complete(mode):
    import torch
    import integer_only_deterministic_amd as D
    if torch.cuda.get_device_properties(0).multi_processor_count < 256:
        pytest.skip("the probe needs 256 CUs")
    print(f"barrier probe mode {mode}", flush=True)
    assert D.detint_probe_barrier(mode, 64) == 0
    assert D.detint_probe_barrier(mode, 0) == 0
