"""The grouped GEMMs' tile schedule on the GPU (moe_debug_schedule), entry
for entry against a plain Python statement of the rule the kernel follows:

  1. tiles of up to bm CSR rows per expert with rows, in expert order, then
     the shared segment's tiles (when the call has one);
  2. tile i (cost 4 + its 32-row token blocks, prefix S_i before it, total C)
     goes to XCD min(7, floor(8 (2 S_i + c_i) / (2 C))): contiguous shares
     of about an eighth of the cost each;
  3. each XCD lists its tiles by class, descending, in tile order within a
     class: the shared segment's tiles (class 9), then every tile of an
     expert with several tiles (class 4, so an expert's tiles stay
     together), then the one-tile experts by token blocks (4, 3, 2, 1);
  4. every entry carries (first row, rows, expert, tiles of its expert,
     record address); sched_n[0] = tiles, sched_n[8 + x] = tiles of XCD x.

The order only decides which workgroup runs which tile (the GEMMs' results do
not depend on it), so these tests pin the schedule itself.  Also: a call
whose tiles exceed the lists' capacity schedules nothing and writes nothing.
"""
import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

COST_BASE = 4


def model(offsets, bm, records, shared):
    """shared: None or (rec, p0, n).  Returns (sched_n[16], lists[8] of tuples)."""
    E = len(offsets) - 1
    segs = [(int(offsets[e]), int(offsets[e + 1]) - int(offsets[e]), e, int(records[e])) for e in range(E)]
    if shared is not None:
        segs.append((shared[1], shared[2], E, shared[0]))
    tiles = []
    for p0, n, e, rec in segs:
        ne = (n + bm - 1) // bm
        for j in range(ne):
            rows = min(bm, n - j * bm)
            tb = (rows + 31) // 32
            cls = 9 if (shared is not None and e == E) else 4 if ne > 1 else tb
            tiles.append(dict(p0=p0 + j * bm, n=rows, expert=e, tiles=ne, rec=rec, tb=tb, cls=cls))
    T = len(tiles)
    C = sum(COST_BASE + t["tb"] for t in tiles)
    S = 0
    for t in tiles:
        c = COST_BASE + t["tb"]
        t["xcd"] = min(7, (8 * (2 * S + c)) // (2 * C))
        S += c
    lists = []
    for x in range(8):
        mine = [t for t in tiles if t["xcd"] == x]
        mine.sort(key=lambda t: -t["cls"])          # stable: tile order within a class
        lists.append([(t["p0"], t["n"], t["expert"], t["tiles"], t["rec"]) for t in mine])
    sched_n = [T] + [0] * 7 + [len(l) for l in lists]
    return sched_n, lists


def run(offsets, bm, records, shared, xcap=None, rows_bound=0):
    import mixture_experts_prefill_amd as mep

    E = len(offsets) - 1
    total_rows = int(offsets[-1] - offsets[0]) + (shared[2] if shared else 0)
    cap = total_rows // 32 + E + 2
    xcap = cap if xcap is None else xcap
    d_off = torch.from_numpy(np.asarray(offsets, np.uint32).view(np.int32)).cuda()
    d_rec = torch.from_numpy(np.asarray(records, np.uint64).view(np.int64)).cuda()
    sched_n = torch.full((16,), -7, dtype=torch.int32, device="cuda")
    # room for 8 full lists of `cap` entries whatever xcap is passed
    order = torch.full((8 * max(cap, xcap) * 8,), -5, dtype=torch.int32, device="cuda")
    mep.moe_debug_schedule(d_off, bm, rows_bound, d_rec, shared[0] if shared else None, shared[1] if shared else 0,
                           shared[2] if shared else 0, sched_n, order, xcap)
    torch.cuda.synchronize()
    sn = sched_n.cpu().numpy().astype(np.int64)
    ent = order.cpu().numpy().reshape(-1, 8)
    return sn, ent, xcap


def check(offsets, bm, records, shared):
    """Both ways the kernel fills its tiles (one thread per segment, or all
    threads with a search: picked by the rows bound) give the model's lists."""
    want_n, want = model(offsets, bm, records, shared)
    for rows_bound in (0, 1 << 20):
        sn, ent, xcap = run(offsets, bm, records, shared, rows_bound=rows_bound)
        assert sn[0] == want_n[0] and list(sn[8:16]) == want_n[8:16], (rows_bound, list(sn), want_n)
        for x in range(8):
            got = []
            for q in range(want_n[8 + x]):
                e = ent[x * xcap + q]
                rec = int(np.array(e[4:6], np.int32).view(np.uint64)[0])
                got.append((int(e[0]), int(e[1]), int(e[2]), int(e[3]), rec))
                assert e[6] == 0 and e[7] == 0
            assert got == want[x], (rows_bound, x)


def random_offsets(rng, E, total, zipf=None, empty=0.3):
    if zipf:
        p = 1.0 / np.arange(1, E + 1) ** zipf
        counts = rng.multinomial(total, p / p.sum())
    else:
        counts = rng.integers(0, max(1, 2 * total // E) + 1, E)
    counts[rng.random(E) < empty] = 0
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)


@pytest.mark.parametrize("bm", [32, 64, 128])
@pytest.mark.parametrize("E", [1, 7, 64, 128, 512, 1024])
def test_schedule_random(bm, E):
    rng = np.random.default_rng(1000 + E + bm)
    records = rng.integers(1, 1 << 47, E, dtype=np.int64).astype(np.uint64) & ~np.uint64(255)
    for trial, total in enumerate((E // 2 + 1, 8 * E, 32768 if E <= 512 else 20000)):
        offsets = random_offsets(rng, E, total, zipf=1.1 if trial == 2 else None)
        check(offsets, bm, records, None)
        t = int(rng.integers(1, 4097))
        check(offsets, bm, records, (0xABCDE00, int(offsets[-1]), t))


def test_schedule_full_chunk_shape():
    """Zipf(1.1) over 128 experts, 32768 positions, the shared segment of
    4096 rows: the full chunk's schedule."""
    rng = np.random.default_rng(5)
    offsets = random_offsets(rng, 128, 32768, zipf=1.1, empty=0.0)
    records = (np.arange(128, dtype=np.uint64) + 1) << np.uint64(20)
    check(offsets, 128, records, (0x7777000, 32768, 4096))


def test_schedule_edge_cases():
    records = (np.arange(64, dtype=np.uint64) + 3) << np.uint64(12)
    empty = np.zeros(65, np.uint32)
    check(empty, 128, records, None)                          # no rows at all: no tiles
    check(empty, 128, records, (0x1000, 0, 8))                # only the shared segment
    one = np.zeros(65, np.uint32)
    one[40:] = 4096                                           # one expert holds every row
    check(one, 128, records, None)
    check(one, 32, records, (0x2000, 4096, 4096))
    exact = np.concatenate([[0], np.cumsum(np.full(64, 128))]).astype(np.uint32)
    check(exact, 128, records, None)                          # every tile full, one class
    check(exact, 64, records, None)


def test_schedule_refuses_lists_too_small():
    """More tiles than the lists hold: sched_n all zero, no entry written."""
    rng = np.random.default_rng(9)
    offsets = random_offsets(rng, 64, 4096, empty=0.0)
    records = np.arange(64, dtype=np.uint64) + 1
    want_n, _ = model(offsets, 32, records, None)
    for rows_bound in (0, 1 << 20):
        sn, ent, xcap = run(offsets, 32, records, None, xcap=want_n[0] - 1, rows_bound=rows_bound)
        assert (sn == 0).all()
        assert (ent == -5).all()
