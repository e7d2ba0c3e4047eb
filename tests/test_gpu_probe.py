"""Device probes through the C ABI.  The HBM read probe (moe_debug_read_probe)
reads its buffer without writing it, and leaves the sink untouched for a
buffer whose per-thread checksums cannot equal the probe's marker value; the
XCC map (moe_debug_xcc_map) shows workgroups whose ids agree modulo 8 on one
XCD."""
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


def test_workgroups_share_an_xcd_by_id_modulo_8():
    """The merged gate/up + down launch keeps a tile's gate/up and down
    workgroups on ids that agree modulo 8 and reads the gate/up rows from
    the L2 of their XCD: this checks that such workgroups share an XCD, over
    more workgroups than fit the device at once."""
    import numpy as np

    import mixture_experts_prefill_amd as mep

    for blocks in (8, 1000, 65536):
        xcc = mep.moe_debug_xcc_map(blocks)
        assert (xcc != 0xffffffff).all()
        ids = np.arange(blocks)
        first = xcc[:min(8, blocks)]
        assert np.array_equal(xcc, first[ids % len(first)]), f"{blocks} workgroups: XCC ids {xcc[:24]}"
    print("XCC ids of workgroups 0-7:", list(mep.moe_debug_xcc_map(8)))
