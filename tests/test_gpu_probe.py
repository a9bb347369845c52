"""The matrix-core ceiling probe used by bench.py: runs through the C ABI,
reports the FLOPs its launch geometry implies, and leaves finite checksums."""
import pytest

pytest.importorskip("torch")
import torch  # noqa: E402

import full_attention_long_amd as ea  # noqa: E402


@pytest.mark.gpu
def test_mfma_probe_runs_and_counts_flops():
    n = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.full((n * 512,), float("nan"), dtype=torch.float32, device="cuda")
    flops = ea.ea_mfma_probe(out, n, 100, seed=7)
    torch.cuda.synchronize()
    assert flops == n * 8 * 100 * 16 * 2 * 32 * 32 * 16
    assert bool(torch.isfinite(out).all())
    # the checksums depend on the seed: the operands are really drawn from it
    out2 = torch.empty_like(out)
    ea.ea_mfma_probe(out2, n, 100, seed=8)
    torch.cuda.synchronize()
    assert not torch.equal(out, out2)
