"""GPU row statistics of a grouped chunk (moe_chunk_stats_fill), the
per-chunk report of the prefill.rs page (struct ChunkStats), bitwise
against a plain numpy reading of the same offsets: tokens, assignments
(offsets[E] - offsets[0]), experts with rows, the most and fewest rows of a
touched expert, and the lower median (position (n - 1) // 2 of the n
non-zero counts sorted ascending).  Cases: a hand example, random counts
with many ties and empty experts at E = 1 .. 1024, a chunk with no rows,
the blocks' own groupings (oracle offsets), and a streamed chunk whose
report carries the ring's fetched records and bytes.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth as ms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

FIELDS = ["tokens", "assignments", "experts_touched", "rows_max", "rows_min", "rows_median"]


@pytest.fixture(scope="module")
def mep():
    import mixture_experts_prefill_amd as m

    m.lib()
    return m


def ref_stats(offsets, t):
    c = np.diff(offsets.astype(np.int64))
    nz = np.sort(c[c > 0])
    n = int(nz.size)
    return dict(tokens=t, assignments=int(offsets[-1]) - int(offsets[0]), experts_touched=n,
                rows_max=int(nz[-1]) if n else 0, rows_min=int(nz[0]) if n else 0,
                rows_median=int(nz[(n - 1) // 2]) if n else 0)


def gpu_stats(mep, offsets, t):
    d_off = torch.from_numpy(offsets.astype(np.uint32).view(np.int32)).cuda()
    stats = torch.full((8,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    mep.moe_chunk_stats_fill(d_off, t, stats)
    torch.cuda.synchronize()
    v = stats.cpu().numpy().view(np.uint32)
    return {f: int(v[i]) for i, f in enumerate(FIELDS)}, v[6:]


def test_hand_example(mep):
    # counts 0, 3, 1, 0, 2, 2: touched 4, sorted 1 2 2 3, lower median 2
    offsets = np.concatenate([[0], np.cumsum([0, 3, 1, 0, 2, 2])]).astype(np.uint32)
    got, pad = gpu_stats(mep, offsets, 4)
    assert got == dict(tokens=4, assignments=8, experts_touched=4, rows_max=3, rows_min=1, rows_median=2)
    assert got == ref_stats(offsets, 4)
    assert (pad == 0).all()


@pytest.mark.parametrize("E", [1, 2, 7, 128, 512, 1000, 1024])
def test_random_counts(mep, E):
    rng = np.random.default_rng(700 + E)
    for trial in range(4):
        counts = rng.integers(0, 6 + 40 * trial, E)
        counts[rng.random(E) < 0.3] = 0
        base = int(rng.integers(0, 1000))       # offsets need not start at 0
        offsets = (base + np.concatenate([[0], np.cumsum(counts)])).astype(np.uint32)
        t = int(rng.integers(0, 4097))
        got, _ = gpu_stats(mep, offsets, t)
        assert got == ref_stats(offsets, t), (E, trial)


def test_no_rows(mep):
    offsets = np.zeros(65, np.uint32)
    got, _ = gpu_stats(mep, offsets, 0)
    assert got == dict(tokens=0, assignments=0, experts_touched=0, rows_max=0, rows_min=0, rows_median=0)


@pytest.mark.parametrize("name", ["tiny", "mid", "decode", "decode1", "full"])
def test_block_report(mep, orc, name):
    """After one moe_block call, the block's report equals the numpy reading
    of the oracle's grouping of the same chunk; nothing is fetched."""
    wl = ms.make_workload(name)
    blk = mep.MoeBlock.from_workload(wl)
    blk.forward(path="block")
    got = blk.chunk_stats()
    lg = orc.router_logits(wl.x, wl.w_router)
    idx, w = orc.topk(lg, wl.cfg.k)
    offsets = orc.build_csr(idx, w, wl.cfg.experts)[0]
    ref = ref_stats(offsets, wl.cfg.t)
    assert {f: got[f] for f in FIELDS} == ref
    assert ref["assignments"] == wl.cfg.t * wl.cfg.k
    assert got["fetched"] == 0 and got["fetched_bytes"] == 0 and got["wait_s"] == 0.0
    print(f"    {name}: {ref}", flush=True)


def test_streamed_report(mep):
    """Streamed experts: the report's fetched records and bytes are the
    ring's (every used expert that is not resident, at the record stride)."""
    seed, t, h, I, E, k, G = 71, 200, 512, 128, 24, 4, 64
    wl = ms.small_case(seed, t, h, I, E, k, G)
    resident = np.zeros(E, dtype=bool)
    resident[::3] = True
    blk = mep.MoeBlock.from_workload(wl, resident=resident, ring_slots=8, group=4)
    blk.forward()
    got = blk.chunk_stats()
    offsets = blk.offsets.cpu().numpy().view(np.uint32)
    used = np.diff(offsets.astype(np.int64)) > 0
    streamed = int((used & ~resident).sum())
    assert {f: got[f] for f in FIELDS} == ref_stats(offsets, t)
    assert got["fetched"] == streamed and streamed > 0
    assert got["fetched_bytes"] == streamed * ms.layout(h, I, G).stride
    assert got["wait_s"] >= 0.0
