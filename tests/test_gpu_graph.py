"""The one-call block under HIP graph capture (the use the no-allocation
entry point is for): moe_block and moe_block_noalloc record no allocation,
memset or host synchronisation, so a captured call replays.  Each graph is
replayed several times, with eager calls on other inputs and
synchronisations between the replays, and every replay is compared bitwise
with the eager call on the same inputs (same kernels, same arithmetic):
logits, routing, grouping and the output.
"""
import numpy as np
import pytest
import torch

import moe_synth as ms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

KEYS = ("logits", "topk_idx", "topk_w", "offsets", "csr_rows", "csr_w", "csr_pos", "out")


def outputs(blk):
    torch.cuda.synchronize()
    return {k: getattr(blk, k).cpu().numpy().copy().view(np.uint32) for k in KEYS}


@pytest.mark.parametrize("entry", ["block", "block_noalloc"])
@pytest.mark.parametrize("name", ["tiny", "decode", "mid"])
def test_graph_replays_match_eager(name, entry):
    import mixture_experts_prefill_amd as mep

    wl = ms.make_workload(name, centred=True)
    blk = mep.MoeBlock.from_workload(wl)
    call = getattr(blk, entry)
    # two input sets: the workload's x and a second, scaled one
    x0 = blk.x.clone()
    x1 = (blk.x.view(torch.bfloat16).float() * 0.5).to(torch.bfloat16).view(blk.x.dtype)
    refs = []
    for xs in (x0, x1):
        blk.x.copy_(xs)
        call(0)
        refs.append(outputs(blk))
    # capture with x0 in place (the graph reads blk.x at replay)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    blk.x.copy_(x0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(0)
    torch.cuda.synchronize()
    for rep in range(4):
        which = rep % 2
        blk.x.copy_(x0 if which == 0 else x1)
        for key in KEYS:
            if key != "out":
                getattr(blk, key).fill_(-1)
        blk.out.fill_(float("nan"))
        g.replay()
        got = outputs(blk)
        for key in KEYS:
            assert np.array_equal(got[key], refs[which][key]), (name, entry, rep, key)
        # eager work between replays, on the other input
        blk.x.copy_(x1 if which == 0 else x0)
        call(0)
        torch.cuda.synchronize()
    del g
