"""The diagnostic matrix-core probe (orbitquant_diag.h): it runs, fills its
sink with finite values, and its flop count follows the documented
formula.  (Its timing is the bench's business.)"""
import numpy as np
import pytest

from tests.gpu_util import host, say

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs():
    import torch
    import quantization_dit_linear_amd as q
    assert torch.cuda.is_available()
    sink = torch.full((3 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    say("mfma probe")
    flop = q.diag_mfma_f16(3, 5, sink)
    torch.cuda.synchronize()
    assert flop == 3 * 8 * 5 * 32 * 16384
    assert np.isfinite(host(sink)).all()
    with pytest.raises(q.OQError):
        q.diag_mfma_f16(0, 5, sink)
