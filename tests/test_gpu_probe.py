"""The MFMA-rate probe (a measurement aid beside the attention path): it runs,
counts its own flops, and every workgroup computes the same sums."""
import pytest
import torch

import block_sparse_attention_07_amd as bsa


@pytest.mark.gpu
def test_mfma_probe_counts_its_flops_and_fills_the_sink():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((512 * cus,), float("nan"), dtype=torch.float32, device="cuda")
    iters = 10
    flops = bsa.mfma_probe(sink, iters)
    torch.cuda.synchronize()
    # two 4-wave workgroups per CU, 16 MFMAs of 32x32x16 (2 flops per term) per iteration
    assert flops == 2 * cus * 4 * iters * 16 * 32 * 32 * 16 * 2
    s = sink.view(2 * cus, 256)
    assert torch.isfinite(s).all()
    assert torch.equal(s, s[:1].expand_as(s))
    with pytest.raises(bsa.BsaError):
        bsa.mfma_probe(sink[: 512 * cus - 1], iters)
