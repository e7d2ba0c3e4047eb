"""GPU parity of streamed experts in the 2-bit miss layout.

Streamed (not resident) experts cross the host link as 2-bit records and are
expanded on the GPU into the 4-bit records the GEMMs read.  Bars:
  - with records built from the same logical codes (0..3) and scale/bias in
    both forms, the ring with 2-bit misses gives bitwise the output of every
    expert resident in 4-bit form, with released slots poisoned or not;
  - against the oracle, which decodes each expert's record in its own form
    (2-bit for the streamed ones): routing bitwise, outputs within the
    block's bar (relative Frobenius error <= 5e-3, max abs <= 1e-2 max), on
    small cases and on every row of the large chunk;
  - the ring's byte counter equals streamed experts x the 2-bit stride.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth as ms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REL_FRO = 5e-3
MAX_ABS_REL = 1e-2


@pytest.fixture(scope="module")
def mep():
    import mixture_experts_prefill_amd as m

    m.lib()
    return m


def check_out(got, ref, what=""):
    ref = np.asarray(ref, dtype=np.float64)
    d = got.astype(np.float64) - ref
    fro = np.linalg.norm(d) / np.linalg.norm(ref)
    mx = np.max(np.abs(d)) / np.max(np.abs(ref))
    print(f"    {what} rows={got.shape[0]} rel_fro={fro:.2e} max_abs_rel={mx:.2e}", flush=True)
    assert fro <= REL_FRO and mx <= MAX_ABS_REL, (fro, mx)


def run(mep, wl, resident, miss_records=None, ring_slots=64, group=8, path=None):
    blk = mep.MoeBlock.from_workload(wl, resident=resident, ring_slots=ring_slots, group=group,
                                     miss_records=miss_records)
    blk.workspace.fill_(0xFF)
    blk.forward(path=path)
    torch.cuda.synchronize()
    g = dict(topk_idx=blk.topk_idx.cpu().numpy().view(np.uint32), offsets=blk.offsets.cpu().numpy().view(np.uint32),
             csr_rows=blk.csr_rows.cpu().numpy().view(np.uint32), out=blk.out.cpu().numpy(),
             stats=blk.ring.stats() if blk.ring is not None else None)
    assert np.isfinite(g["out"]).all()
    del blk
    return g


def twin_records(seed, L4, L2, E, centred):
    """Per expert, the same logical codes (0..3) and fp16 scale/bias packed
    as a 4-bit record and as a 2-bit record."""
    rng = np.random.default_rng(seed)
    r4 = np.zeros((E, L4.stride), np.uint8)
    r2 = np.zeros((E, L2.stride), np.uint8)
    for e in range(E):
        mats = {}
        for m in ("gate", "up", "down"):
            N, K = ms.matrix_shape(L4, m)
            s = rng.uniform(0.025, 0.1, (N, K // L4.group)).astype(np.float16)
            b = rng.normal(0, 0.01, (N, K // L4.group)).astype(np.float16)
            if centred:
                b = (b - 1.5 * s.astype(np.float64)).astype(np.float16)
            mats[m] = (rng.integers(0, 4, (N, K)), s, b)
        r4[e] = ms.pack_record(L4, mats)
        r2[e] = ms.pack_record(L2, mats, bits=2)
    return r4, r2


SMALL = [
    # seed, t, h, I, E, k, G
    (60, 200, 512, 128, 24, 4, 64),
    (61, 64, 256, 192, 40, 6, 32),
    (62, 8, 1024, 256, 64, 8, 64),     # few-row tiles of streamed experts
    (63, 600, 768, 128, 16, 2, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}-t{c[1]}-h{c[2]}-I{c[3]}-E{c[4]}-k{c[5]}" for c in SMALL])
def test_lowbit_misses_small(mep, orc, case):
    seed, t, h, I, E, k, G = case
    wl = ms.small_case(seed, t, h, I, E, k, G, centred=True)
    L4 = ms.layout(h, I, G)
    L2 = ms.layout(h, I, G, 2)
    r4, r2 = twin_records(seed, L4, L2, E, centred=True)
    wl = dataclasses.replace(wl, records=r4)
    resident = np.zeros(E, dtype=bool)
    resident[::3] = True
    base = run(mep, wl, None, path="separate")               # every expert resident, 4-bit
    g = run(mep, wl, resident, miss_records=r2, ring_slots=8, group=4)
    assert np.array_equal(g["out"], base["out"]), "2-bit misses differ from the same codes resident in 4-bit form"
    streamed = int(((np.diff(g["offsets"].astype(np.int64)) > 0) & ~resident).sum())
    assert g["stats"]["streamed"] == streamed and g["stats"]["fetched_bytes"] == streamed * L2.stride
    bits = np.where(resident, 4, 2).astype(np.uint8)
    mixed = r4.copy()
    mixed[~resident, :L2.stride] = r2[~resident]
    ref = orc.block(dataclasses.replace(wl, records=mixed), record_bits=bits, with_logits=False)
    assert np.array_equal(g["topk_idx"], ref["topk_idx"]) and np.array_equal(g["csr_rows"], ref["csr_rows"])
    check_out(g["out"], ref["out"], "2-bit misses")


def test_lowbit_misses_with_poisoned_slots(mep, monkeypatch):
    """Released ring and staging slots filled with 0xFF before their next
    copy: no bit of the output may change."""
    seed, t, h, I, E, k, G = 64, 300, 512, 128, 30, 4, 64
    wl = ms.small_case(seed, t, h, I, E, k, G, centred=True)
    L4, L2 = ms.layout(h, I, G), ms.layout(h, I, G, 2)
    r4, r2 = twin_records(seed, L4, L2, E, centred=True)
    wl = dataclasses.replace(wl, records=r4)
    resident = np.zeros(E, dtype=bool)
    resident[::7] = True
    base = run(mep, wl, resident, miss_records=r2, ring_slots=4, group=2)
    monkeypatch.setenv("MOE_RING_POISON", "1")
    g = run(mep, wl, resident, miss_records=r2, ring_slots=4, group=2)
    assert np.array_equal(g["out"], base["out"])


@pytest.mark.timeout(900)
def test_lowbit_misses_large(mep, orc):
    """The large chunk: top-64 experts by rows resident in 4-bit form, the
    other 448 streamed as 2-bit records; every row against the oracle."""
    wl = ms.make_workload("large", centred=True)
    print("  oracle routing ...", flush=True)
    lg = orc.router_logits(wl.x, wl.w_router)
    idx, w = orc.topk(lg, wl.cfg.k)
    offsets = orc.build_csr(idx, w, wl.cfg.experts)[0]
    resident = orc.residency(offsets, wl.cfg.resident)
    streamed_ids = np.nonzero(~resident)[0]
    L2 = ms.layout(wl.cfg.hidden, wl.cfg.inter, wl.cfg.group, 2)
    miss = np.zeros((wl.cfg.experts, L2.stride), np.uint8)
    miss[streamed_ids] = ms.make_records(wl.cfg, experts=streamed_ids.tolist(), centred=True, bits=2)
    print("  GPU ring with 2-bit misses ...", flush=True)
    g = run(mep, wl, resident, miss_records=miss)
    used = np.diff(offsets.astype(np.int64)) > 0
    assert g["stats"]["streamed"] == int((used & ~resident).sum())
    assert g["stats"]["fetched_bytes"] == g["stats"]["streamed"] * L2.stride
    assert np.array_equal(g["topk_idx"], idx) and np.array_equal(g["offsets"], offsets)
    bits = np.where(resident, 4, 2).astype(np.uint8)
    wl.records[streamed_ids, :L2.stride] = miss[streamed_ids]    # the oracle reads each record in its own form
    print("  oracle block ...", flush=True)
    ref = orc.block(wl, record_bits=bits, with_logits=False)
    check_out(g["out"], ref["out"], "large, 2-bit misses")
