"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (the block's acceptance criteria):
  - topk_idx, offsets, csr_rows, csr_pos: bitwise equal to the oracle;
  - topk_w, csr_w: within 1e-6 absolute of the oracle, and csr_w bitwise
    equal to the GPU's own topk_w at the same (row, expert);
  - block output: relative Frobenius error <= 5e-3 and
    max |gpu - ref| <= 1e-2 * max |ref| (bf16 activations and weights,
    fp32 accumulation, against the oracle's double result).
Every test also compares the router logits bitwise with the oracle's fixed
fp32 summation order.  The five workloads run at their own shapes with both
the plain weights and the centred ones (bias = -7.5 scale + noise, so the
weights are near zero mean and the Frobenius check is not dominated by the
mean component); every output row is compared with the oracle's grouped
block.
"""
import os

import numpy as np
import pytest
import torch

import moe_synth as ms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REL_FRO = 5e-3
MAX_ABS_REL = 1e-2
W_ABS = 1e-6


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def mep():
    import mixture_experts_prefill_amd as m

    m.lib()
    return m


def run(mep, wl, resident=None, ring_slots=64, group=8, shared=True, force_ring=False, path=None):
    """One block; `path` None takes forward()'s default (moe_block whenever
    every expert is resident), else "block", "fused" (moe_route,
    moe_build_csr, moe_prefill_fused) or "separate" (moe_shared +
    moe_prefill_experts)."""
    blk = mep.MoeBlock.from_workload(wl, resident=resident, ring_slots=ring_slots, group=group, shared=shared)
    if force_ring:
        blk.use_ring(ring_slots, group)
    if path == "fused":
        assert blk.can_fuse
    # NaN bytes in every intermediate: a GEMM tile or feature block that the
    # schedule skipped would leave NaN rows in the output.
    blk.workspace.fill_(0xFF)
    blk.forward(path=path)
    torch.cuda.synchronize()
    g = dict(
        logits=blk.logits.cpu().numpy(),
        topk_idx=blk.topk_idx.cpu().numpy().view(np.uint32),
        topk_w=blk.topk_w.cpu().numpy(),
        offsets=blk.offsets.cpu().numpy().view(np.uint32),
        csr_rows=blk.csr_rows.cpu().numpy().view(np.uint32),
        csr_w=blk.csr_w.cpu().numpy(),
        csr_pos=blk.csr_pos.cpu().numpy().view(np.uint32),
        out=blk.out.cpu().numpy(),
    )
    g["ring_stats"] = blk.ring.stats() if blk.ring is not None else None
    assert np.isfinite(g["out"]).all(), "non-finite outputs: some rows were never computed"
    del blk
    return g


def check_routing(g, r):
    if "logits" in r:
        same = g["logits"].view(np.uint32) == r["logits"].view(np.uint32)
        assert same.all(), f"{int((~same).sum())} router logits differ from the oracle's fp32 order"
    assert np.array_equal(g["topk_idx"], r["topk_idx"]), "top-k indices differ"
    assert np.max(np.abs(g["topk_w"] - r["topk_w"])) <= W_ABS
    assert np.array_equal(g["offsets"], r["offsets"]), "offsets differ"
    assert np.array_equal(g["csr_rows"], r["csr_rows"]), "csr_rows differ"
    assert np.array_equal(g["csr_pos"], r["csr_pos"]), "csr_pos differ"
    assert np.max(np.abs(g["csr_w"] - r["csr_w"])) <= W_ABS
    assert np.array_equal(g["csr_w"][g["csr_pos"]], g["topk_w"].reshape(-1)), "csr_w is not the GPU's topk_w"


def check_out(got, ref, tag=None):
    ref = np.asarray(ref, dtype=np.float64)
    d = got.astype(np.float64) - ref
    fro = np.linalg.norm(d) / np.linalg.norm(ref)
    mx = np.max(np.abs(d)) / np.max(np.abs(ref))
    line = f"{'PARITY ' + tag + ' ' if tag else ''}rows={got.shape[0]} rel_fro={fro:.2e} max_abs_rel={mx:.2e}"
    say("    " + line)
    if tag and os.environ.get("MOE_PARITY_LOG"):
        with open(os.environ["MOE_PARITY_LOG"], "a") as f:
            f.write(line + "\n")
    assert fro <= REL_FRO and mx <= MAX_ABS_REL, (fro, mx)


_REF = {}


def workload_ref(orc, name, centred):
    """The oracle's whole block (every row) for one of the five workloads,
    computed once per (workload, weights) and shared by the paths."""
    key = (name, centred)
    if key not in _REF:
        wl = ms.make_workload(name, centred=centred)
        say(f"  oracle {name} centred={centred} ...")
        _REF.clear()   # keep one at a time: the large workload's result is 64 MiB
        _REF[key] = orc.block(wl)
        del wl
    return _REF[key]


# ------------------------------------------------------------------ small shapes, full oracle

PATHS = ["block", "fused", "separate"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("centred", [False, True])
def test_tiny_config(mep, orc, centred, path):
    wl = ms.make_workload("tiny", centred=centred)
    g = run(mep, wl, path=path)
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])


SWEEP = [
    # seed, t, h, I, E, k, G, centred, gate
    (0, 1, 256, 64, 1, 1, 64, False, False),
    (1, 7, 256, 128, 4, 2, 32, True, False),
    (2, 33, 512, 192, 16, 3, 64, True, True),
    (3, 64, 256, 64, 64, 10, 32, False, False),
    (4, 65, 768, 128, 8, 8, 64, True, False),     # k = E: dense softmax mixture
    (5, 40, 256, 256, 33, 5, 64, False, True),
    (6, 129, 512, 128, 12, 4, 32, True, False),   # several M-tiles per expert, ragged tail
    (7, 300, 256, 64, 3, 2, 64, True, False),     # > 100 rows per expert
    (8, 16, 1024, 320, 30, 6, 32, True, True),    # inter not a multiple of 128
    (9, 161, 256, 64, 37, 4, 64, True, False),    # LDS router tile with ragged rows and experts
    (10, 130, 768, 128, 96, 6, 32, False, False), # LDS router, 3 steps of 256
    (11, 3, 8192, 128, 64, 4, 64, False, False),  # t <= 8 with h > 4096: tiled router; wide few-row rows
    (12, 5, 256, 64, 130, 7, 32, True, True),     # few-row router with t < 8 and E % 4 != 0
    (13, 2, 512, 192, 9, 2, 32, False, False),    # few-row router, 2 rows
    (14, 8, 1024, 256, 300, 10, 64, True, False), # decode-like: ~1 row per expert, E % 64 != 0
    (15, 200, 512, 128, 16, 6, 64, True, True),   # 64-row tiles, forked shared expert, 64-thread combine
    (17, 64, 256, 64, 1024, 32, 32, True, False), # the expert and top-k caps: E = 1024, k = 32
    (18, 4096, 256, 64, 64, 32, 64, False, True), # the row cap with k = 32: 131072 CSR entries
    (22, 4000, 256, 64, 1024, 8, 64, True, False),# 63 CSR tiles (ragged last) with E = 1024 counts each
    (23, 1000, 256, 64, 300, 4, 32, False, False),# 32 x 32 LDS router tiles with ragged rows and experts
    (24, 2, 4096, 256, 12, 3, 64, True, False),   # few-row gate/up launch (waves split K), two-row tiles
    (25, 1, 8192, 320, 40, 5, 32, False, True),   # few-row gate/up launch, 32 K steps per wave, gated
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", SWEEP, ids=[f"s{c[0]}-t{c[1]}-h{c[2]}-I{c[3]}-E{c[4]}-k{c[5]}" for c in SWEEP])
def test_small_sweep(mep, orc, case, path):
    seed, t, h, I, E, k, G, centred, gate = case
    wl = ms.small_case(seed, t, h, I, E, k, G, centred=centred, with_gate=gate)
    g = run(mep, wl, path=path)
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])


TIE_CASES = [(1, 64, 4), (8, 512, 10), (8, 1024, 16), (16, 130, 8), (100, 300, 12), (100, 128, 8), (600, 64, 6)]


@pytest.mark.parametrize("path", ["block", "separate"])
@pytest.mark.parametrize("kind", ["zero", "dup7"])
@pytest.mark.parametrize("case", TIE_CASES, ids=[f"t{c[0]}-E{c[1]}-k{c[2]}" for c in TIE_CASES])
def test_routing_ties(mep, orc, case, kind, path):
    """Exactly equal logits: the selection order is logit descending, then
    expert id ascending.  "zero": W_r = 0, every logit is +0 and the top-k is
    experts 0..k-1 with weights 1/k.  "dup7": router row e repeats row e % 7,
    so each row has 7 distinct logits, each held by about E/7 experts (ties
    across lanes, and within a lane once E > 448)."""
    import dataclasses

    t, E, k = case
    wl = ms.small_case(900 + E, t, 256, 64, E, k, 32)
    if kind == "zero":
        w = np.zeros_like(wl.w_router)
    else:
        w = np.ascontiguousarray(wl.w_router[np.arange(E) % 7])
    wl = dataclasses.replace(wl, w_router=w)
    g = run(mep, wl, path=path)
    r = orc.block(wl)
    check_routing(g, r)
    if kind == "zero":
        assert np.array_equal(g["topk_idx"], np.tile(np.arange(k, dtype=np.uint32), (t, 1)))
    check_out(g["out"], r["out"])


EXTREME_CASES = [(8, 1024, 32), (16, 1000, 32), (100, 1024, 32), (1, 1024, 1), (16, 1, 1), (17, 777, 31),
                 (5, 300, 7), (6, 513, 9), (7, 64, 3)]


@pytest.mark.parametrize("path", ["block", "separate"])
@pytest.mark.parametrize("case", EXTREME_CASES, ids=[f"t{c[0]}-E{c[1]}-k{c[2]}" for c in EXTREME_CASES])
def test_routing_extremes(mep, orc, case, path):
    """The largest expert count and k the calls accept (E = 1024, k = 32),
    partly filled key slots (E = 1000, 777), a single expert, the row
    counts around the merged decode kernel's limit (16 / 17 rows), and 5-7
    rows (the few-row router's two waves per expert, one partly filled)."""
    t, E, k = case
    wl = ms.small_case(950 + E + k, t, 256, 64, E, k, 32)
    g = run(mep, wl, path=path)
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])


def random_cases(n, seed=7):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        t = int(rng.choice([1, 2, 3, 8, 17, 64, 65, 130, 257, 600]))
        h = int(rng.choice([256, 512, 768, 1024]))
        I = int(rng.choice([64, 128, 192, 320]))
        E = int(rng.integers(1, 300))
        k = int(rng.integers(1, min(E, 12) + 1))
        G = int(rng.choice([32, 64]))
        cases.append((100 + i, t, h, I, E, k, G, bool(rng.integers(2)), bool(rng.integers(2))))
    return cases


RANDOM = random_cases(12)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", RANDOM, ids=[f"r{c[0]}-t{c[1]}-h{c[2]}-I{c[3]}-E{c[4]}-k{c[5]}-G{c[6]}" for c in RANDOM])
def test_random_shapes(mep, orc, case, path):
    """Seeded random shapes (row counts around the tile and CSR-tile edges,
    any E and k, both group sizes, gated or not) on every path."""
    seed, t, h, I, E, k, G, centred, gate = case
    wl = ms.small_case(seed, t, h, I, E, k, G, centred=centred, with_gate=gate)
    g = run(mep, wl, path=path)
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])


@pytest.mark.parametrize("t", [1, 8, 100])
def test_shared_of_another_shape(mep, orc, t):
    """A shared expert whose inter differs from the routed one cannot join the
    routed launches: forward() takes the separate calls."""
    wl = ms.small_case(19, t, 512, 128, 12, 3, 64, inter_shared=192, centred=True, with_gate=t == 8)
    blk = mep.MoeBlock.from_workload(wl)
    assert not blk.can_fuse
    del blk
    g = run(mep, wl)
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])


def test_fused_matches_separate(mep):
    """The two paths add the same terms in the same order; they differ only in
    the shared expert's output being rounded to bf16 on the fused path."""
    wl = ms.small_case(20, 150, 512, 128, 24, 4, 64, centred=True, with_gate=True)
    a = run(mep, wl, path="fused")
    b = run(mep, wl, path="separate")
    for key in ("topk_idx", "offsets", "csr_rows", "csr_pos"):
        assert np.array_equal(a[key], b[key]), key
    check_out(a["out"], b["out"].astype(np.float64))


def test_fork_matches_one_stream(mep):
    """The shared expert on a second stream (fork) or first on the same
    stream gives the same bits: the order of additions into out is the same."""
    wl = ms.small_case(16, 100, 512, 128, 24, 4, 64, centred=True, with_gate=True)
    outs = []
    for fork in (True, False):
        blk = mep.MoeBlock.from_workload(wl)
        blk.workspace.fill_(0xFF)
        blk.forward(fork=fork, fused=False)
        torch.cuda.synchronize()
        outs.append(blk.out.cpu().numpy())
        del blk
    assert np.array_equal(outs[0], outs[1])


def test_max_rows_small_dims(mep, orc):
    """t = 4096 (the row cap) at small hidden size: CSR tiles of 64 rows, max tiles."""
    wl = ms.small_case(9, 4096, 256, 64, 16, 4, 64, centred=True)
    g = run(mep, wl)
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])


def test_no_shared_expert(mep, orc):
    wl = ms.small_case(10, 50, 256, 128, 6, 2, 64, centred=True)
    g = run(mep, wl, shared=False)
    r = orc.block(wl, shared_expert=False)
    check_routing(g, r)
    check_out(g["out"], r["out"])


# ------------------------------------------------------------------ the five workloads

WEIGHTS = [False, True]
WEIGHT_IDS = ["plain", "centred"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("centred", WEIGHTS, ids=WEIGHT_IDS)
def test_mid_config(mep, orc, path, centred):
    wl = ms.make_workload("mid", centred=centred)
    g = run(mep, wl, path=path)
    r = workload_ref(orc, "mid", centred)
    check_routing(g, r)
    check_out(g["out"], r["out"], f"mid {WEIGHT_IDS[centred]} {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("centred", WEIGHTS, ids=WEIGHT_IDS)
@pytest.mark.parametrize("name", ["decode", "decode1"])
def test_decode_configs(mep, orc, name, path, centred):
    wl = ms.make_workload(name, centred=centred)
    g = run(mep, wl, path=path)
    r = workload_ref(orc, name, centred)
    check_routing(g, r)
    check_out(g["out"], r["out"], f"{name} {WEIGHT_IDS[centred]} {path}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("centred", WEIGHTS, ids=WEIGHT_IDS)
def test_full_config(mep, orc, path, centred):
    """The full chunk (4096 rows, Zipf routing): every row against the oracle."""
    wl = ms.make_workload("full", centred=centred)
    g = run(mep, wl, path=path)
    del wl
    r = workload_ref(orc, "full", centred)
    check_routing(g, r)
    check_out(g["out"], r["out"], f"full {WEIGHT_IDS[centred]} {path}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("centred", WEIGHTS, ids=WEIGHT_IDS)
def test_large_config(mep, orc, centred):
    """The large chunk: top-64 experts by row count resident and the rest
    streamed through a 64-slot ring in batches of 8; then every expert
    resident on the separate calls (bitwise equal to the ring) and on the
    one-call block.  Every row of each against the oracle."""
    wl = ms.make_workload("large", centred=centred)
    r = workload_ref(orc, "large", centred)
    resident = orc.residency(r["offsets"], wl.cfg.resident)
    say("  GPU ring ...")
    g = run(mep, wl, resident=resident)
    check_routing(g, r)
    st = g["ring_stats"]
    n_streamed = int(((np.diff(r["offsets"].astype(np.int64)) > 0) & ~resident).sum())
    assert st["streamed"] == n_streamed and st["fetched_bytes"] == n_streamed * wl.layout.stride
    check_out(g["out"], r["out"], f"large {WEIGHT_IDS[centred]} ring")
    say("  GPU all resident, separate calls ...")
    g_res = run(mep, wl, path="separate")
    assert np.array_equal(g["out"], g_res["out"]), "ring output differs from all-resident output"
    del g_res
    say("  GPU all resident, one-call block ...")
    g_blk = run(mep, wl, path="block")
    del wl
    check_routing(g_blk, r)
    check_out(g_blk["out"], r["out"], f"large {WEIGHT_IDS[centred]} block")


def test_bruteforce_sample_rows(mep, orc):
    """Sampled rows of the full chunk against the oracle's per-token path,
    which never builds the CSR (a second route to the same reference)."""
    wl = ms.make_workload("full", centred=True)
    g = run(mep, wl)
    rng = np.random.default_rng(1)
    s = np.unique(np.concatenate([[0, wl.cfg.t - 1], rng.choice(wl.cfg.t, 40, replace=False)])).astype(np.int32)
    ref = orc.tokens_bruteforce(wl, s)
    check_out(g["out"][s], ref)


# ------------------------------------------------------------------ invariants of the GPU path

def test_ring_equals_resident_with_poison(mep, monkeypatch):
    """A small ring (4 slots, batches of 2) with released slots poisoned must not change a bit."""
    wl = ms.make_workload("mid")
    base = run(mep, wl, path="separate")
    resident = np.zeros(wl.cfg.experts, dtype=bool)
    resident[::5] = True
    monkeypatch.setenv("MOE_RING_POISON", "1")
    g = run(mep, wl, resident=resident, ring_slots=4, group=2)
    assert np.array_equal(g["out"], base["out"])
    monkeypatch.setenv("MOE_RING_POISON", "0")
    monkeypatch.setenv("MOE_RING_DELAY_US", "200")
    g2 = run(mep, wl, resident=resident, ring_slots=8, group=4)
    assert np.array_equal(g2["out"], base["out"])


def test_ring_with_everything_resident(mep):
    wl = ms.make_workload("tiny")
    a = run(mep, wl, path="separate")
    b = run(mep, wl, force_ring=True, ring_slots=2, group=1)
    assert np.array_equal(a["out"], b["out"])


WAIT_CASES = [
    (31, 256, 8192, 128, 8, 1, 64),   # one gate/up workgroup per tile over 128 K steps; a tile's 32 down workgroups wait
    (32, 96, 4096, 256, 4, 2, 32),    # three tiles, each of two gate/up and sixteen down workgroups
]


@pytest.mark.parametrize("case", WAIT_CASES, ids=[f"t{c[1]}-h{c[2]}-I{c[3]}-E{c[4]}-k{c[5]}" for c in WAIT_CASES])
def test_merged_launch_waits(mep, orc, case):
    """Chunks whose down workgroups reach their tile long before its gate/up
    workgroups finish (few tiles per XCD, long K): the merged gate/up + down
    launch (moe_prefill_experts on resident experts) against the oracle and
    bitwise against the ring's separate gate/up and down launches."""
    seed, t, h, I, E, k, G = case
    wl = ms.small_case(seed, t, h, I, E, k, G, centred=True)
    g = run(mep, wl, path="separate")
    b = run(mep, wl, force_ring=True, ring_slots=8, group=2)
    assert np.array_equal(g["out"], b["out"]), "merged launch differs from the two launches"
    r = orc.block(wl)
    check_routing(g, r)
    check_out(g["out"], r["out"])
    blk = run(mep, wl, path="block")
    check_out(blk["out"], r["out"])


def test_merged_launch_gives_up_visibly(mep, orc):
    """A tile wait that cannot complete, forced from the host (one completion
    more than a tile's gate/up workgroups can give, at most 16 polls): every
    down workgroup of the merged launch takes its give-up path and writes NaN
    in place of its outputs, so every output row is NaN and every launch
    ends.  The normal settings then give the oracle's result again."""
    wl = ms.small_case(32, 96, 4096, 256, 4, 2, 32, centred=True)
    r = orc.block(wl)
    blk = mep.MoeBlock.from_workload(wl)
    # zero intermediates: without the give-up writes every output would be finite
    blk.workspace.zero_()
    try:
        mep.moe_debug_tile_wait(16, 1)
        blk.forward(path="block")
        torch.cuda.synchronize()
    finally:
        mep.moe_debug_tile_wait(0, 0)
    bad = blk.out.cpu().numpy()
    del blk
    assert np.isnan(bad).all(), f"{int(np.isfinite(bad).sum())} outputs finite after a failed wait"
    good = run(mep, wl, path="block")
    check_out(good["out"], r["out"])


@pytest.mark.parametrize("path", PATHS)
def test_deterministic(mep, path):
    wl = ms.small_case(11, 200, 512, 128, 16, 4, 64, centred=True)
    a = run(mep, wl, path=path)
    b = run(mep, wl, path=path)
    for key in ("topk_idx", "topk_w", "offsets", "csr_rows", "csr_w", "csr_pos", "out"):
        assert np.array_equal(a[key], b[key]), key


def test_fused_accumulate(mep, orc):
    """moe_prefill_fused: accumulate=0 overwrites whatever out holds (NaN
    here), accumulate=1 adds the whole block onto it."""
    wl = ms.small_case(21, 40, 256, 128, 8, 3, 64, centred=True, with_gate=True)
    blk = mep.MoeBlock.from_workload(wl)
    blk.workspace.fill_(0xFF)
    blk.route()
    blk.build_csr()
    blk.out.fill_(float("nan"))
    blk.fused(accumulate=0)
    torch.cuda.synchronize()
    first = blk.out.cpu().numpy()
    r = orc.block(wl)
    check_out(first, r["out"])
    blk.out.fill_(1.0)
    blk.fused(accumulate=1)
    torch.cuda.synchronize()
    check_out(blk.out.cpu().numpy(), r["out"] + 1.0)
    # the one-call block, same semantics
    blk.out.fill_(float("nan"))
    blk.block(accumulate=0)
    torch.cuda.synchronize()
    check_out(blk.out.cpu().numpy(), r["out"])
    blk.out.fill_(1.0)
    blk.block(accumulate=1)
    torch.cuda.synchronize()
    check_out(blk.out.cpu().numpy(), r["out"] + 1.0)


def test_accumulate_semantics(mep, orc):
    wl = ms.small_case(12, 24, 256, 128, 8, 2, 64, centred=True)
    blk = mep.MoeBlock.from_workload(wl)
    blk.out.fill_(float("nan"))
    blk.shared(accumulate=0)
    shared_only = blk.out.clone()
    blk.route()
    blk.build_csr()
    blk.out.fill_(float("nan"))
    blk.experts(accumulate=0)
    experts_only = blk.out.clone()
    blk.out.copy_(shared_only)
    blk.experts(accumulate=1)
    torch.cuda.synchronize()
    assert torch.isfinite(shared_only).all() and torch.isfinite(experts_only).all()
    ys = orc.shared(wl.shared_record, 256, 128, 64, wl.x)
    check_out(shared_only.cpu().numpy(), ys)
    r = orc.block(wl)
    check_out(blk.out.cpu().numpy(), r["out"])
    r0 = orc.block(wl, shared_expert=False)
    check_out(experts_only.cpu().numpy(), r0["out"])


@pytest.mark.parametrize("name,t", [("decode", 8), ("decode", 1), ("mid", 64), ("mid", 200)])
def test_shared_expert_gate(mep, orc, name, t):
    """The shared expert alone with its sigmoid gate, on chunks that split K
    over workgroups (t <= 64, partial sums reduced in a fixed order) and on a
    chunk that does not; accumulate=1 adds onto what out holds."""
    wl = ms.make_workload(name, centred=True, with_gate=True, t=t)
    c = wl.cfg
    blk = mep.MoeBlock.from_workload(wl)
    blk.workspace.fill_(0xFF)
    blk.out.fill_(float("nan"))
    blk.shared(accumulate=0)
    torch.cuda.synchronize()
    got = blk.out.cpu().numpy()
    ref = orc.shared(wl.shared_record, c.hidden, c.inter_shared, c.group, wl.x, wl.gate_w)
    check_out(got, ref)
    blk.out.fill_(1.0)
    blk.shared(accumulate=1)
    torch.cuda.synchronize()
    check_out(blk.out.cpu().numpy(), ref + 1.0)


def test_bad_arguments_leave_outputs_untouched(mep):
    wl = ms.make_workload("tiny")
    blk = mep.MoeBlock.from_workload(wl)
    blk.out.fill_(7.0)
    blk.topk_idx.fill_(-1)
    with pytest.raises(mep.MoeError) as e:
        mep.moe_route(blk.x, blk.w_router, 9, blk.logits, blk.topk_idx, blk.topk_w)   # k > E
    assert e.value.status == 1
    with pytest.raises(mep.MoeError) as e:
        mep.moe_prefill_experts(blk.x, 2, 8, blk.L, blk.offsets, blk.csr_rows, blk.csr_w, blk.csr_pos, blk.table,
                                blk.out, 1, blk.workspace[:1024])
    assert e.value.status == 3
    table = blk.table.clone()
    table[3] = 0                                  # expert 3 not resident, no ring
    blk.route()
    blk.build_csr()
    torch.cuda.synchronize()
    if int(blk.offsets[4] - blk.offsets[3]) > 0:
        ring_slots = torch.empty((4, blk.L.stride), dtype=torch.uint8, device="cuda")
        ring = mep.MoeRing(blk.L, ring_slots, 4, 2)
        with pytest.raises(mep.MoeError):
            mep.moe_prefill_experts(blk.x, 2, 8, blk.L, blk.offsets, blk.csr_rows, blk.csr_w, blk.csr_pos, table,
                                    blk.out, 1, blk.workspace, host_records=[None] * 8, ring=ring)
        ring.close()
    torch.cuda.synchronize()
    assert bool((blk.out == 7.0).all())


def test_missing_record_does_not_fault(mep):
    """A used expert whose record address is 0 (and no ring) is never
    dereferenced: its entries get unspecified values, every other row is
    unchanged, on every path."""
    wl = ms.small_case(24, 64, 256, 128, 8, 2, 64, centred=True)
    for path in PATHS:
        ref = run(mep, wl, path=path)
        blk = mep.MoeBlock.from_workload(wl)
        blk.workspace.fill_(0xFF)
        blk.route()
        blk.build_csr()
        torch.cuda.synchronize()
        table = blk.table.clone()
        table[3] = 0
        blk.table = table
        if path == "block":
            blk.block(accumulate=0)
        elif path == "fused":
            blk.fused(accumulate=0)
        else:
            blk.shared(accumulate=0)
            blk.experts(accumulate=1)
        torch.cuda.synchronize()
        out = blk.out.cpu().numpy()
        idx = blk.topk_idx.cpu().numpy()
        clean = ~(idx == 3).any(axis=1)
        assert clean.any() and (~clean).any()
        assert np.array_equal(out[clean], ref["out"][clean])
        del blk
