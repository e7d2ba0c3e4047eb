"""Host-side tests of the C ABI: no GPU needed, no kernel is launched.

Checks that libmoe loads and exports every symbol its headers declare, that
its record layout and workspace plan agree with the independent copies in the
generator and the oracle, that argument validation returns the right status
before anything is enqueued, and that the expert ring's host schedule keeps
the slot-reuse rule of the experts.rs page (fn pf_experts).
"""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import moe_synth as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
mep = pytest.importorskip("mixture_experts_prefill_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mep.LIB_PATH):
        from mixture_experts_prefill_amd import build

        build.build()
    return mep.lib()


def header_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(moe_[a-z_0-9]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert {"moe_route", "moe_build_csr", "moe_prefill_experts", "moe_shared"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(mep.EXPORTS) >= names


@pytest.mark.parametrize("h,I,G", [(256, 128, 32), (2048, 768, 64), (4096, 1536, 64), (512, 192, 32)])
def test_layout_agrees_with_generator_and_oracle(lib, orc, h, I, G):
    L = mep.moe_layout_make(h, I, G).as_dict()
    g = ms.layout(h, I, G)
    o = orc.layout(h, I, G)
    for k in ("gate_w", "gate_sb", "up_w", "up_sb", "down_w", "down_sb", "stride"):
        assert L[k] == getattr(g, k) == o[k], k
    assert L["bits"] == 4 and L["hidden"] == h and L["inter"] == I and L["group"] == G


@pytest.mark.parametrize("h,I,G", [(128, 64, 64), (256, 96, 64), (256, 128, 16), (0, 64, 64)])
def test_layout_rejects_bad_shapes(lib, h, I, G):
    with pytest.raises(mep.MoeError) as e:
        mep.moe_layout_make(h, I, G)
    assert e.value.status == 1


def test_workspace_plan(lib):
    L = mep.moe_layout_make(2048, 768, 64)
    Ls = mep.moe_layout_make(2048, 768, 64)
    t, k, E = 4096, 8, 128
    n = mep.moe_workspace_bytes(t, k, E, L, Ls)
    P = t * k
    # hg and ye (bf16) dominate: with a shared expert of the routed layout they
    # hold t more rows (moe_prefill_fused), plus the shared scratch t*Is*2
    Q = P + t
    assert n >= Q * 768 * 2 + Q * 2048 * 2 + t * 768 * 2
    assert n < Q * 768 * 2 + Q * 2048 * 2 + t * 768 * 2 + 8 * 2**20
    assert n % 256 == 0
    # no shared expert, or one of another shape: t*k rows only
    n0 = mep.moe_workspace_bytes(t, k, E, L, None)
    assert P * 768 * 2 + P * 2048 * 2 <= n0 < P * 768 * 2 + P * 2048 * 2 + 8 * 2**20
    Ls2 = mep.moe_layout_make(2048, 1536, 64)
    n2 = mep.moe_workspace_bytes(t, k, E, L, Ls2)
    assert n2 < P * 768 * 2 + P * 2048 * 2 + t * 1536 * 2 + 8 * 2**20
    assert mep.moe_workspace_bytes(0, k, E, L, Ls) == 0
    assert mep.moe_workspace_bytes(4097, k, E, L, Ls) == 0
    assert mep.moe_workspace_bytes(t, 9, 8, L, Ls) == 0


def P(v):
    return ctypes.c_void_p(v)


FAKE = 1 << 20  # never dereferenced: validation fails before any use


@pytest.mark.parametrize("t,h,E,k,status", [
    (0, 256, 8, 2, 2),       # empty chunk
    (4097, 256, 8, 2, 2),    # over the row cap
    (16, 255, 8, 2, 1),      # h not a multiple of 256
    (16, 256, 8, 9, 1),      # k > E
    (16, 256, 0, 1, 1),      # no experts
    (16, 256, 2048, 2, 1),   # too many experts
    (16, 256, 64, 33, 1),    # k above the cap
])
def test_route_validation(lib, t, h, E, k, status):
    rc = lib.moe_route(P(FAKE), P(FAKE), t, h, E, k, P(FAKE), P(FAKE), P(FAKE), None)
    assert rc == status
    assert lib.moe_last_error().decode()


def test_null_and_alignment_checks(lib):
    assert lib.moe_route(None, P(FAKE), 16, 256, 8, 2, P(FAKE), P(FAKE), P(FAKE), None) == 1
    assert lib.moe_route(P(FAKE + 2), P(FAKE), 16, 256, 8, 2, P(FAKE), P(FAKE), P(FAKE), None) == 1
    L = mep.moe_layout_make(256, 128, 32)
    assert lib.moe_shared(P(FAKE), 16, ctypes.byref(L), None, None, P(FAKE), 0, P(FAKE), 1 << 20, None) == 1
    bad = mep.moe_layout_make(256, 128, 32)
    bad.stride += 1
    assert lib.moe_shared(P(FAKE), 16, ctypes.byref(bad), P(FAKE), None, P(FAKE), 0, P(FAKE), 1 << 20, None) == 1
    assert lib.moe_shared(P(FAKE), 0, ctypes.byref(L), P(FAKE), None, P(FAKE), 0, P(FAKE), 1 << 20, None) == 2


def test_32bit_offset_limits(lib):
    """The GEMMs address records, x and the intermediate rows with 32-bit byte
    offsets; shapes beyond that are refused before anything is enqueued."""
    with pytest.raises(mep.MoeError) as e:
        mep.moe_layout_make(65536, 65536, 64)          # three 2 GiB code sections
    assert e.value.status == 1 and "4 GiB" in e.value.message
    L = mep.moe_layout_make(256, 16384, 64)            # t*k*I*2 = 4096*32*16384*2 = 4 GiB
    rc = lib.moe_prefill_experts(P(FAKE), 4096, 32, 64, ctypes.byref(L), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                 P(FAKE), None, None, P(FAKE), 1, P(FAKE), 1 << 40, None)
    assert rc == 2 and "32-bit" in lib.moe_last_error().decode()
    Ls = mep.moe_layout_make(256, 524352, 64)          # t*Is*2 > 4 GiB at t = 4096
    rc = lib.moe_shared(P(FAKE), 4096, ctypes.byref(Ls), P(FAKE), None, P(FAKE), 0, P(FAKE), 1 << 40, None)
    assert rc == 2 and "32-bit" in lib.moe_last_error().decode()


def test_workspace_too_small(lib):
    L = mep.moe_layout_make(256, 128, 32)
    need = mep.moe_workspace_bytes(16, 2, 8, L, L)
    assert lib.moe_build_csr(P(FAKE), P(FAKE), 4096, 8, 1024, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1024,
                             None) == 3
    assert lib.moe_shared(P(FAKE), 16, ctypes.byref(L), P(FAKE), None, P(FAKE), 0, P(FAKE), 256, None) == 3
    assert lib.moe_prefill_experts(P(FAKE), 16, 2, 8, ctypes.byref(L), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                   None, None, P(FAKE), 1, P(FAKE), need // 4, None) == 3


def test_ring_create_validation(lib):
    L = mep.moe_layout_make(256, 128, 32)
    h = ctypes.c_void_p()
    assert lib.moe_ring_create(ctypes.byref(L), P(FAKE), 4, 8, ctypes.byref(h)) == 1   # slots < group
    assert lib.moe_ring_create(ctypes.byref(L), P(FAKE), 12, 8, ctypes.byref(h)) == 1  # not a multiple
    assert lib.moe_ring_create(ctypes.byref(L), None, 64, 8, ctypes.byref(h)) == 1


# ------------------------------------------------------------------ ring schedule simulator

def random_offsets(rng, E, t, k, empty_frac):
    counts = rng.integers(1, 50, E)
    counts[rng.random(E) < empty_frac] = 0
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("n_slots,group", [(64, 8), (8, 2), (16, 16), (6, 3)])
def test_ring_schedule_reuse_rule(lib, seed, n_slots, group):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 400))
    offsets = random_offsets(rng, E, 0, 0, rng.random() * 0.5)
    resident = (rng.random(E) < rng.random()).astype(np.uint64)
    slot, batch, wait = mep.moe_ring_plan_debug(offsets, resident, n_slots, group)
    counts = np.diff(offsets.astype(np.int64))
    jobs = [e for e in range(E) if counts[e] > 0]
    # jobs in ascending id, consecutive batches of `group`
    assert [batch[e] for e in jobs] == [i // group for i in range(len(jobs))]
    assert all(batch[e] == -1 and slot[e] == -1 for e in range(E) if counts[e] == 0)
    streamed = [e for e in jobs if not resident[e]]
    assert [slot[e] for e in streamed] == [i % n_slots for i in range(len(streamed))]
    assert all(slot[e] == -1 for e in jobs if resident[e])
    lag = n_slots // group
    assert list(wait) == [b - lag if b >= lag else -1 for b in range(len(wait))]
    # reuse rule: when a slot is taken again, the new user's batch waits for a
    # batch at or after the previous user's batch (so the previous user is done)
    last_user = {}
    for e in streamed:
        s, b = slot[e], batch[e]
        if s in last_user:
            prev_b = last_user[s]
            assert prev_b < b
            assert wait[b] >= prev_b
        last_user[s] = b


def test_fused_validation(lib):
    """moe_prefill_fused refuses a shared layout other than the routed one, null
    pointers, a short workspace and shapes beyond its 32-bit offsets, all before
    anything is enqueued."""
    L = mep.moe_layout_make(256, 128, 32)
    Ls_other = mep.moe_layout_make(256, 192, 32)
    need = mep.moe_workspace_bytes(16, 2, 8, L, L)
    args = lambda Ls, rec, ws: (P(FAKE), 16, 2, 8, ctypes.byref(L), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                ctypes.byref(Ls), rec, None, P(FAKE), 0, P(FAKE), ws, None)
    assert lib.moe_prefill_fused(*args(Ls_other, P(FAKE), need)) == 1
    assert "must equal" in lib.moe_last_error().decode()
    assert lib.moe_prefill_fused(*args(L, None, need)) == 1
    assert lib.moe_prefill_fused(*args(L, P(FAKE + 8), need)) == 1          # misaligned record
    assert lib.moe_prefill_fused(*args(L, P(FAKE), need - 256)) == 3
    # the shared rows follow the t*k routed rows: t*(k+1)*I*2 > 4 GiB is refused
    Lb = mep.moe_layout_make(256, 16384, 64)
    rc = lib.moe_prefill_fused(P(FAKE), 4096, 31, 64, ctypes.byref(Lb), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                               P(FAKE), ctypes.byref(Lb), P(FAKE), None, P(FAKE), 0, P(FAKE), 1 << 40, None)
    assert rc == 2 and "32-bit" in lib.moe_last_error().decode()


def test_block_validation(lib):
    """moe_block validates like the separate calls, before anything is enqueued."""
    L = mep.moe_layout_make(256, 128, 32)
    Lo = mep.moe_layout_make(256, 192, 32)
    need = mep.moe_workspace_bytes(16, 2, 8, L, L)

    def call(t=16, k=2, E=8, Ls=L, ws=need, w_router=P(FAKE), rec=P(FAKE)):
        return lib.moe_block(P(FAKE), w_router, t, k, E, ctypes.byref(L), P(FAKE),
                             ctypes.byref(Ls) if Ls is not None else None, rec, None,
                             P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                             P(FAKE), 0, P(FAKE), ws, None)

    assert call(t=0) == 2 and "empty chunk" in lib.moe_last_error().decode()
    assert call(k=9) == 1
    assert call(Ls=Lo) == 1 and "must equal" in lib.moe_last_error().decode()
    assert call(w_router=None) == 1
    assert call(w_router=P(FAKE + 4)) == 1                 # misaligned router weights
    assert call(rec=None) == 1                             # shared layout without a record
    assert call(ws=need - 256) == 3
    # without a shared expert the workspace of the routed experts alone suffices
    assert call(Ls=None, rec=None, ws=mep.moe_workspace_bytes(16, 2, 8, L, None) - 256) == 3


def test_block_noalloc_refuses_beyond_its_scratch(lib):
    """moe_block_noalloc checks the chunk's scratch against its static
    64 MiB before touching the device: the full chunk (about 204 MiB) is
    refused, as are the argument errors moe_block refuses."""
    L = mep.moe_layout_make(2048, 768, 64)
    assert mep.moe_workspace_bytes(4096, 8, 128, L, L) > mep.NOALLOC_SCRATCH_BYTES

    def call(t=4096, k=8, E=128, w_router=P(FAKE)):
        return lib.moe_block_noalloc(P(FAKE), w_router, t, k, E, ctypes.byref(L), P(FAKE), ctypes.byref(L), P(FAKE),
                                     None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                     0, None)

    assert call() == 2 and "scratch" in lib.moe_last_error().decode()
    assert call(t=0) == 2 and "empty chunk" in lib.moe_last_error().decode()
    assert call(k=200) == 1
    assert call(w_router=None) == 1


def test_next_norm_validation(lib):
    """moe_inject_norm and moe_block_next_norm refuse bad descriptions of the
    residual copies before anything is enqueued."""
    t, h = 16, 256
    hyper, gamma, mixed = FAKE, FAKE + (1 << 20), FAKE + (2 << 20)

    def nn(n=2, eps=1e-6, hy=hyper, gm=gamma, mx=mixed):
        d = mep.moe_next_norm()
        d.hyper, d.n, d.gamma, d.eps, d.mixed = hy, n, gm, eps, mx
        return d

    def inj(d, y=None, tt=t, hh=h):
        return lib.moe_inject_norm(y, tt, hh, ctypes.byref(d), None)

    assert inj(nn(n=0)) == 1 and inj(nn(n=17)) == 1
    assert inj(nn(eps=-1.0)) == 1 and inj(nn(eps=float("inf"))) == 1
    assert inj(nn(hy=None)) == 1 and inj(nn(gm=None)) == 1 and inj(nn(mx=None)) == 1
    assert inj(nn(mx=mixed + 8)) == 1                                  # misaligned
    assert inj(nn(), hh=200) == 1 and inj(nn(), hh=16640) == 1         # h % 256, h > 16384
    assert inj(nn(mx=hyper + 4096)) == 1                               # mixed inside the copies
    assert "overlap" in lib.moe_last_error().decode()
    assert inj(nn(), y=P(hyper + 256)) == 1                            # y inside the copies
    assert inj(nn(), tt=0) == 2 and inj(nn(), tt=4097) == 2
    assert lib.moe_inject_norm(None, t, h, None, None) == 1
    L = mep.moe_layout_make(h, 128, 32)
    need = mep.moe_workspace_bytes(t, 2, 8, L, L)

    def blk(d, ws=need):
        return lib.moe_block_next_norm(P(FAKE), P(FAKE), t, 2, 8, ctypes.byref(L), P(FAKE), ctypes.byref(L),
                                       P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                       ctypes.byref(d) if d is not None else None, P(FAKE), ws, None)

    assert blk(None) == 1
    assert blk(nn(n=0)) == 1
    assert blk(nn(), ws=need - 256) == 3
    assert blk(nn(mx=hyper)) == 1


def test_chunk_stats_validation(lib):
    """moe_chunk_stats_fill refuses bad arguments before anything is enqueued."""
    f = lib.moe_chunk_stats_fill
    assert f(P(FAKE), 16, 0, P(FAKE), None) == 1
    assert f(P(FAKE), 16, 1025, P(FAKE), None) == 1
    assert f(P(FAKE), -1, 8, P(FAKE), None) == 1
    assert f(None, 16, 8, P(FAKE), None) == 1
    assert f(P(FAKE), 16, 8, None, None) == 1
    assert f(P(FAKE), 16, 8, P(FAKE + 2), None) == 1                   # stats misaligned
    assert "aligned" in lib.moe_last_error().decode()


def test_read_probe_validation(lib):
    """moe_debug_read_probe refuses bad arguments without launching."""
    f = lib.moe_debug_read_probe
    assert f(None, 1 << 20, 64, P(FAKE), None) == 1
    assert f(P(FAKE), 1 << 20, 64, None, None) == 1
    assert f(P(FAKE + 8), 1 << 20, 64, P(FAKE), None) == 1              # src misaligned
    assert f(P(FAKE), (1 << 20) + 4, 64, P(FAKE), None) == 1            # not whole 16-byte loads
    assert f(P(FAKE), 1 << 20, 0, P(FAKE), None) == 1
    assert f(P(FAKE), 1 << 20, 65537, P(FAKE), None) == 1


def test_xcc_map_validation(lib):
    """moe_debug_xcc_map refuses bad arguments without launching."""
    f = lib.moe_debug_xcc_map
    assert f(None, 8, None) == 1
    assert f(P(FAKE), 0, None) == 1
    assert f(P(FAKE), (1 << 20) + 1, None) == 1


def test_tile_wait_validation(lib):
    """moe_debug_tile_wait accepts its documented range only, and 0, 0
    restores normal operation."""
    f = lib.moe_debug_tile_wait
    assert f(-1, 0) == 1
    assert f(32769, 0) == 1
    assert f(0, -1) == 1
    assert f(0, 2) == 1
    assert f(16, 1) == 0
    assert f(32768, 0) == 0
    assert f(0, 0) == 0


def test_schedule_debug_validation(lib):
    """moe_debug_schedule refuses bad arguments without launching."""
    f = lib.moe_debug_schedule
    ok = dict(off=P(FAKE), E=8, bm=128, rb=4096, rec=P(FAKE), srec=None, sp0=0, sn=0, sched=P(FAKE),
              order=P(FAKE), xcap=64)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["off"], a["E"], a["bm"], a["rb"], a["rec"], a["srec"], a["sp0"], a["sn"], a["sched"],
                 a["order"], a["xcap"], None)

    assert call(off=None) == 1 and call(rec=None) == 1 and call(sched=None) == 1 and call(order=None) == 1
    assert call(E=0) == 1 and call(E=1025) == 1
    assert call(bm=48) == 1 and call(bm=256) == 1
    assert call(xcap=0) == 1 and call(rb=-1) == 1
    assert call(sp0=-1) == 1 and call(sn=-1) == 1
    assert call(srec=P(FAKE), sn=0) == 1                               # a shared record needs rows
