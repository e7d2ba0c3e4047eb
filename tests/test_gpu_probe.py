"""The HBM read probe (moe_debug_read_probe) runs through the C ABI, reads
its buffer without writing it, and leaves the sink untouched for a buffer
whose per-thread checksums cannot equal the probe's marker value."""
import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_read_probe_runs():
    import mixture_experts_prefill_amd as mep

    src = torch.arange(1 << 22, dtype=torch.int32, device="cuda")   # 16 MiB
    before = src.clone()
    for blocks in (1, 7, 4096):
        sink = torch.full((blocks,), 5, dtype=torch.int32, device="cuda")
        mep.moe_debug_read_probe(src, blocks, sink)
        torch.cuda.synchronize()
        assert torch.equal(src, before)
        # every word is below 2^22, so no thread's XOR can equal the marker
        # (0x9E3779B9): nothing is stored
        assert (sink == 5).all()
