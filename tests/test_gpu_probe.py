"""The MFMA-loop probe (a measurement helper beside the decode path): every
thread's sum of its four accumulation chains is exactly 64 * iters (each
32x32x16 MFMA on operands of ones adds 16 to every accumulator element)."""
import pytest
import torch

import decode_attention_11_amd as mla
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (256, 37), (1024, 500)])
def test_probe_mfma_computes_exact_sums(workgroups, iters):
    say(f"probe {workgroups} x {iters}")
    out = mla.probe_mfma(workgroups, iters)
    torch.cuda.synchronize()
    assert out.numel() == workgroups * 256
    assert torch.equal(out, torch.full_like(out, 64.0 * iters))
