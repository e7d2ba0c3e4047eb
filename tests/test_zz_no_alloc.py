"""moe_block_noalloc (the one-call block on the library's static scratch)
against moe_block with a caller's workspace, through the C ABI.

Two calls in a row, the second with a smaller chunk, so the second finds the
first call's contents in the scratch; each is compared with moe_block on the
same inputs (same kernels: bitwise equal) and with the oracle (the block's
tolerance).  Collected last: its file name sorts after every other test.
"""
import numpy as np
import pytest
import torch

import moe_synth as ms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REL_FRO = 5e-3
MAX_ABS_REL = 1e-2
KEYS = ("logits", "topk_idx", "topk_w", "offsets", "csr_rows", "csr_w", "csr_pos", "out")


def outputs(blk):
    torch.cuda.synchronize()
    return {k: getattr(blk, k).cpu().numpy().copy() for k in KEYS}


def check_out(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    d = got.astype(np.float64) - ref
    fro = np.linalg.norm(d) / np.linalg.norm(ref)
    mx = np.max(np.abs(d)) / np.max(np.abs(ref))
    print(f"    rows={got.shape[0]} rel_fro={fro:.2e} max_abs_rel={mx:.2e}", flush=True)
    assert fro <= REL_FRO and mx <= MAX_ABS_REL, (fro, mx)


@pytest.mark.parametrize("name,rows", [("mid", (512, 100)), ("decode", (8, 1))])
def test_noalloc_matches_block(name, rows, orc):
    import mixture_experts_prefill_amd as mep

    for t in rows:
        print(f"  {name}: t = {t}", flush=True)
        wl = ms.make_workload(name, centred=True, t=t)
        blk = mep.MoeBlock.from_workload(wl)
        assert mep.moe_workspace_bytes(t, wl.cfg.k, wl.cfg.experts, blk.L, blk.Ls) <= mep.NOALLOC_SCRATCH_BYTES
        blk.workspace.fill_(0xFF)
        blk.out.fill_(float("nan"))
        blk.block(accumulate=0)
        ref = outputs(blk)
        for key in KEYS:
            getattr(blk, key).fill_(-1)
        blk.block_noalloc(accumulate=0)
        got = outputs(blk)
        for key in KEYS:
            assert np.array_equal(got[key].view(np.uint32), ref[key].view(np.uint32)), key
        # accumulate = 1 adds onto what out holds
        blk.out.fill_(1.0)
        blk.block_noalloc(accumulate=1)
        acc = outputs(blk)["out"]
        r = orc.block(wl)
        assert np.array_equal(got["topk_idx"].view(np.uint32), r["topk_idx"])
        assert np.array_equal(got["csr_rows"].view(np.uint32), r["csr_rows"])
        check_out(got["out"], r["out"])
        check_out(acc, r["out"].astype(np.float64) + 1.0)
        del blk


def test_noalloc_rejects_a_chunk_beyond_its_scratch():
    """The full chunk needs about 204 MiB of scratch: refused before
    anything runs, outputs untouched."""
    import mixture_experts_prefill_amd as mep

    wl = ms.make_workload("full")
    blk = mep.MoeBlock.from_workload(wl)
    blk.out.fill_(7.0)
    with pytest.raises(mep.MoeError) as e:
        blk.block_noalloc(accumulate=0)
    assert e.value.status == 2 and "scratch" in e.value.message
    torch.cuda.synchronize()
    assert bool((blk.out == 7.0).all())
