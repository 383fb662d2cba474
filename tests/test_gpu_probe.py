"""The MFMA rate probe that the bench reports beside the published peak: it runs, zero operands
give zero checksums, random ones finite and non-zero ones."""
import pytest
import torch

import ring_attention_merge_amd as ram

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs():
    out = torch.full((4 * 512,), float("nan"), device="cuda")
    ram.mfma_probe(4, 3, 0, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))
    ram.mfma_probe(4, 3, 1, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out != 0).any()
