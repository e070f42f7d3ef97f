"""The calibration launch (register-resident matrix ops on random operands) runs on the GPU,
writes its sink and reports the launch's operation count."""
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,per_op", [(ssn.PROBE_BF16, 2 * 32 * 32 * 16), (ssn.PROBE_FP4, 2 * 32 * 32 * 64)])
@pytest.mark.parametrize("wps", [1, 2])
def test_mfma_probe_runs(kind, per_op, wps):
    sink = torch.full((ssn.mfma_probe_sink_floats(),), float("nan"), dtype=torch.float32, device="cuda")
    flops = ssn.mfma_probe(kind, wps, 8, sink, seed=3)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == per_op * (16 if wps == 1 else 8) * 8 * cus * wps * 4
    written = sink[: cus * wps * 256]
    assert bool(torch.isfinite(written).all())
