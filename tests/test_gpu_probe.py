"""GPU check of the matrix-core rate probe that bench.py reports beside the nominal peak:
it runs through the C ABI and returns the accumulator sums (finite, and equal on two runs
since every workgroup does the same arithmetic)."""
import pytest
import torch

import tree_causal_draft_amd as jt
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def test_probe_runs_and_is_deterministic():
    need_gpu()
    out = jt.probe_mfma_rate(16, 8)
    torch.cuda.synchronize()
    a = out.clone()
    jt.probe_mfma_rate(16, 8, out)
    torch.cuda.synchronize()
    assert out.shape == (8 * 256,)
    assert torch.isfinite(out).all() and torch.equal(a, out)
