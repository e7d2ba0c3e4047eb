"""Pins of the CPU oracle against facts fixed outside it.

Each test ties one oracle function to a closed form, a library routine
(numpy / torch float64), an invariant the pages state, or a hand-derived
fixture, so that a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a wrong order) fails at least one of them.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import moe_synth as ms

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24


def bf16(a):
    return ms.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def xf(xbits):
    return ms.bf16_bits_to_f32(xbits).astype(np.float64)


# ------------------------------------------------------------------ record format

def test_layout_matches_generator_and_sizes(orc):
    for h, I, G in [(256, 128, 32), (2048, 768, 64), (4096, 1536, 64), (512, 192, 32)]:
        a = orc.layout(h, I, G)
        b = ms.layout(h, I, G)
        for k, v in a.items():
            assert v == getattr(b, k), (h, I, G, k)
    # record bytes R = 3*h*I*(1/2 + 4/G), already 4096-aligned at these shapes
    assert orc.layout(2048, 768, 64)["stride"] == 2_654_208
    assert orc.layout(4096, 1536, 64)["stride"] == 10_616_832
    assert orc.layout(256, 128, 32)["stride"] == 61_440


def test_dequant_codes_only(orc):
    """scale = 1, bias = 0 -> W = q exactly (pins code positions)."""
    h, I, G = 256, 128, 32
    L = ms.layout(h, I, G)
    g = np.random.default_rng(1)
    mats = {}
    for m in ("gate", "up", "down"):
        N, K = ms.matrix_shape(L, m)
        mats[m] = (g.integers(0, 16, (N, K)), np.ones((N, K // G)), np.zeros((N, K // G)))
    rec = ms.pack_record(L, mats)
    for m in ("gate", "up", "down"):
        W = orc.dequant(rec, m, h, I, G)
        assert np.array_equal(W, mats[m][0].astype(np.float64)), m


def test_dequant_hand_placed_byte(orc):
    """One byte written by hand from the stated format decodes to the stated positions.

    Tile (ob=1, kb=2) of gate (K = h = 256 -> 4 tiles per row block), lane 33,
    word 2, byte 2 = 0x5A: word 2 holds codes c = 16..23; byte 2 holds bits
    16..23 = code c%8=1 (bits 16-19) and c%8=3 (bits 20-23).  So row
    32*1 + 33%32 = 33, columns 64*2 + 32 + 17 = 177 (q = 0xA) and 179 (q = 5).
    """
    h, I, G = 256, 128, 64
    L = ms.layout(h, I, G)
    rec = np.zeros(L.stride, dtype=np.uint8)
    tile = 1 * (h // 64) + 2
    rec[L.gate_w + tile * 1024 + 16 * 33 + 4 * 2 + 2] = 0x5A
    # scale 1.0 (0x3C00), bias 0 for every entry of the gate sb section
    nent = I * h // G
    sb = np.zeros(nent, dtype=np.uint32) | 0x3C00
    rec[L.gate_sb: L.gate_sb + 4 * nent] = sb.astype("<u4").view(np.uint8)
    W = orc.dequant(rec, "gate", h, I, G)
    nz = np.argwhere(W != 0)
    assert nz.tolist() == [[33, 177], [33, 179]]
    assert W[33, 177] == 10.0 and W[33, 179] == 5.0


@pytest.mark.parametrize("G", [32, 64])
def test_dequant_scale_bias_per_group(orc, G):
    """q = 0 -> W = bias of the group; dyadic scale 2^-4 with codes -> exact s*q + b."""
    h, I = 256, 64
    L = ms.layout(h, I, G)
    g = np.random.default_rng(2)
    mats = {}
    for m in ("gate", "up", "down"):
        N, K = ms.matrix_shape(L, m)
        s = np.full((N, K // G), 2.0 ** -4)
        b = g.integers(-64, 64, (N, K // G)) * 2.0 ** -8
        q = np.zeros((N, K), dtype=np.int64) if m == "gate" else g.integers(0, 16, (N, K))
        mats[m] = (q, s, b)
    rec = ms.pack_record(L, mats)
    for m in ("gate", "up", "down"):
        q, s, b = mats[m]
        W = orc.dequant(rec, m, h, I, G)
        expect = np.repeat(b, G, axis=1) + np.repeat(s, G, axis=1) * q
        assert np.array_equal(W, expect), m
    # q = 0: every column of a group equals that group's bias
    Wg = orc.dequant(rec, "gate", h, I, G)
    assert np.array_equal(Wg[:, ::G], mats["gate"][2])


def test_f16_decode_special_values(orc):
    """fp16 subnormal, negative, and max decode exactly (scale = value, q = 1, bias = 0)."""
    h, I, G = 64, 64, 64
    L = ms.layout(h, I, G)
    vals = np.array([2.0 ** -24, -2.0 ** -14, 65504.0, -0.5, 1.0 + 2.0 ** -10], dtype=np.float16)
    mats = {}
    for m in ("gate", "up", "down"):
        N, K = ms.matrix_shape(L, m)
        s = np.resize(vals, (N, K // G)).astype(np.float16)
        mats[m] = (np.ones((N, K), dtype=np.int64), s, np.zeros((N, K // G), dtype=np.float16))
    rec = ms.pack_record(L, mats)
    W = orc.dequant(rec, "up", h, I, G)
    assert np.array_equal(W[:, 0], mats["up"][1][:, 0].astype(np.float64))


# ------------------------------------------------------------------ router

def test_router_golden_order(orc):
    with open(os.path.join(GOLDEN, "router_order.json")) as f:
        cases = json.load(f)["cases"]
    h = 256
    x = bf16(np.ones((1, h)))
    for c in cases:
        w = np.zeros((1, h), dtype=np.float32)
        for i, v in c["w"].items():
            w[0, int(i)] = v
        got = orc.router_logits(x, w)[0, 0]
        assert got == c["canonical"] and not np.signbit(got), c["name"]
        # the fixture's 'sequential' value really is the left-to-right float32 sum
        acc = np.float32(0)
        for i in range(h):
            acc = np.float32(acc + w[0, i])
        assert acc == c["sequential"], c["name"]


def test_router_zero_and_one_hot(orc):
    h, E = 512, 7
    g = np.random.default_rng(3)
    w = g.normal(0, 0.02, (E, h)).astype(np.float32)
    lz = orc.router_logits(bf16(g.normal(0, 1, (3, h))), np.zeros((E, h), np.float32))
    assert np.all(lz == 0) and not np.any(np.signbit(lz))
    for i in (0, 3, 255, 256, 511):
        x = np.zeros((1, h), np.float32)
        x[0, i] = 1.0
        assert np.array_equal(orc.router_logits(bf16(x), w)[0], w[:, i])


def test_router_exact_on_dyadic_inputs(orc):
    """Small integers times multiples of 2^-4 sum exactly in any order: equals the float64 matmul."""
    h, E, t = 1024, 9, 5
    g = np.random.default_rng(4)
    x = g.integers(-8, 9, (t, h)).astype(np.float32)
    w = (g.integers(-16, 17, (E, h)) / 16.0).astype(np.float32)
    got = orc.router_logits(bf16(x), w)
    assert np.array_equal(got.astype(np.float64), x.astype(np.float64) @ w.T.astype(np.float64))


@pytest.mark.parametrize("h", [256, 2048, 4096])
def test_router_error_bound(orc, h):
    """|fp32 canonical - exact| <= (h/64 + 6) * 2^-24 * sum|x_i w_i| (fmaf chains of h/64, 6 tree levels)."""
    g = np.random.default_rng(h)
    xb = bf16(g.normal(0, 1, (8, h)))
    w = g.normal(0, 0.02, (16, h)).astype(np.float32)
    got = orc.router_logits(xb, w).astype(np.float64)
    x = xf(xb)
    exact = x @ w.T.astype(np.float64)
    bound = (h / 64 + 6) * U * (np.abs(x) @ np.abs(w.T.astype(np.float64))) * 1.0001
    assert np.all(np.abs(got - exact) <= bound)


# ------------------------------------------------------------------ top-k

def ref_topk(lg, k):
    """Library stable sort: descending logit, ties to lower id."""
    order = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")
    return order[:, :k]


def test_topk_matches_stable_sort(orc):
    g = np.random.default_rng(5)
    lg = g.normal(0, 1, (200, 64)).astype(np.float32)
    lg[::7, 3] = lg[::7, 10]          # exact ties
    lg[::11, 5] = -0.0
    lg[::11, 6] = 0.0                 # -0 vs +0 tie
    for k in (1, 2, 8, 64):
        idx, w = orc.topk(lg, k)
        assert np.array_equal(idx, ref_topk(lg, k))
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= k * U * 2)


def test_topk_ties_and_special_k(orc):
    E = 12
    idx, w = orc.topk(np.zeros((3, E), np.float32), 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1)))
    assert np.all(w == np.float32(0.25))
    g = np.random.default_rng(6)
    lg = g.normal(0, 2, (50, E)).astype(np.float32)
    idx, w = orc.topk(lg, E)
    assert all(sorted(r) == list(range(E)) for r in idx.tolist())
    idx1, w1 = orc.topk(lg, 1)
    assert np.all(w1 == 1.0)
    # k = 2 closed form: w1 = 1 / (1 + exp(l2 - l1))
    idx2, w2 = orc.topk(lg, 2)
    l1 = lg[np.arange(50), idx2[:, 0]].astype(np.float64)
    l2 = lg[np.arange(50), idx2[:, 1]].astype(np.float64)
    assert np.allclose(w2[:, 0], 1 / (1 + np.exp(l2 - l1)), rtol=0, atol=1e-7)


def test_topk_is_softmax_then_renormalise(orc):
    """Equals torch softmax over all E (float64), top-k, divided by the selected mass."""
    g = np.random.default_rng(7)
    lg = g.normal(0, 1.5, (40, 32)).astype(np.float32)
    idx, w = orc.topk(lg, 6)
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=1).numpy()
    sel = np.take_along_axis(p, idx.astype(np.int64), 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=0, atol=2e-7)


# ------------------------------------------------------------------ grouping

def check_csr_invariants(idx, w, E, offsets, rows, cw, pos):
    t, k = idx.shape
    counts = np.diff(offsets.astype(np.int64))
    assert offsets[0] == 0 and offsets[-1] == t * k and np.all(counts >= 0)
    assert np.array_equal(np.bincount(rows, minlength=t), np.full(t, k))     # each row exactly k times
    for e in range(E):
        seg = rows[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg.astype(np.int64)) > 0)                      # stable, distinct
        assert np.array_equal(np.sort(seg), np.nonzero((idx == e).any(1))[0])
    flat = idx.reshape(-1)
    assert np.array_equal(rows[pos], np.repeat(np.arange(t), k))             # inverse map
    assert np.array_equal(np.searchsorted(offsets, pos, side="right") - 1, flat)
    assert np.array_equal(cw[pos], w.reshape(-1))


def test_csr_matches_stable_sort_and_invariants(orc):
    g = np.random.default_rng(8)
    for t, E, k in [(1, 4, 2), (33, 16, 3), (300, 64, 8), (64, 8, 8)]:
        lg = g.normal(0, 1, (t, E)).astype(np.float32)
        idx, w = orc.topk(lg, k)
        offsets, rows, cw, pos = orc.build_csr(idx, w, E)
        check_csr_invariants(idx, w, E, offsets, rows, cw, pos)
        flat = idx.reshape(-1).astype(np.int64)
        order = np.argsort(flat, kind="stable")       # library stable sort of (e, r)
        assert np.array_equal(rows, order // k)
        assert np.array_equal(cw, w.reshape(-1)[order])


def test_residency_stable_by_count(orc):
    offsets = np.cumsum([0, 5, 0, 7, 5, 1, 7, 0, 2]).astype(np.uint32)
    keep = orc.residency(offsets, 3)
    counts = np.diff(offsets)
    ranked = sorted([e for e in range(8) if counts[e]], key=lambda e: -counts[e])
    assert set(np.nonzero(keep)[0]) == set(ranked[:3]) == {2, 5, 0}


# ------------------------------------------------------------------ expert FFN and block

def torch_swiglu(orc, rec, h, I, G, x64):
    Wg = torch.from_numpy(orc.dequant(rec, "gate", h, I, G))
    Wu = torch.from_numpy(orc.dequant(rec, "up", h, I, G))
    Wd = torch.from_numpy(orc.dequant(rec, "down", h, I, G))
    X = torch.from_numpy(x64)
    a = torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)
    return (a @ Wd.T).numpy()


def test_expert_ffn_is_textbook_swiglu(orc):
    wl = ms.small_case(0, 24, 256, 192, 1, 1, 32, centred=True)
    y = orc.expert_rows(wl.records[0], 256, 192, 32, wl.x, list(range(24)))
    ref = torch_swiglu(orc, wl.records[0], 256, 192, 32, xf(wl.x))
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_zero_gate_gives_zero_output(orc):
    h, I, G = 128, 64, 64
    L = ms.layout(h, I, G)
    g = np.random.default_rng(9)
    mats = {}
    for m in ("gate", "up", "down"):
        N, K = ms.matrix_shape(L, m)
        z = (m == "gate")
        mats[m] = (g.integers(0, 16, (N, K)), np.zeros((N, K // G)) if z else g.uniform(0.005, 0.02, (N, K // G)),
                   np.zeros((N, K // G)) if z else g.normal(0, 0.01, (N, K // G)))
    rec = ms.pack_record(L, mats)
    x = bf16(g.normal(0, 1, (4, h)))
    assert np.all(orc.expert_rows(rec, h, I, G, x, [0, 1, 2, 3]) == 0)


def test_shared_expert_and_gate(orc):
    wl = ms.small_case(1, 12, 256, 128, 2, 1, 64, centred=True)
    ref = torch_swiglu(orc, wl.shared_record, 256, 128, 64, xf(wl.x))
    ys = orc.shared(wl.shared_record, 256, 128, 64, wl.x)
    assert np.max(np.abs(ys - ref)) <= 1e-12 * np.max(np.abs(ref))
    half = orc.shared(wl.shared_record, 256, 128, 64, wl.x, gate_w=np.zeros(256, np.uint16))
    assert np.array_equal(half, 0.5 * ys)                       # sigmoid(0) = 1/2 exactly
    gw = bf16(np.random.default_rng(10).normal(0, 0.05, 256))
    gated = orc.shared(wl.shared_record, 256, 128, 64, wl.x, gate_w=gw)
    z = xf(wl.x) @ xf(gw)
    assert np.allclose(gated, ys * torch.sigmoid(torch.from_numpy(z)).numpy()[:, None], rtol=1e-12, atol=0)


@pytest.mark.parametrize("centred", [False, True])
def test_block_grouped_equals_bruteforce(orc, centred):
    """Grouped path == per-token sum in ascending expert id (bitwise after rounding); slot order within 1e-12."""
    wl = ms.small_case(2, 40, 256, 128, 8, 3, 32, centred=centred)
    r = orc.block(wl)
    check_csr_invariants(r["topk_idx"], r["topk_w"], 8, r["offsets"], r["csr_rows"], r["csr_w"], r["csr_pos"])
    bf = orc.tokens_bruteforce(wl, list(range(40)), order=0)
    assert np.array_equal(bf.astype(np.float32), r["out"])
    bf1 = orc.tokens_bruteforce(wl, list(range(40)), order=1)
    assert np.max(np.abs(bf1 - bf)) <= 1e-12 * np.max(np.abs(bf))
    # routing outputs of the block equal the separate calls
    lg = orc.router_logits(wl.x, wl.w_router)
    idx, w = orc.topk(lg, 3)
    assert np.array_equal(idx, r["topk_idx"]) and np.array_equal(w, r["topk_w"])


def test_dense_limit_is_softmax_mixture(orc):
    """k = E: out = shared + sum_e softmax(logits)_e * FFN_e(x), with torch float64 library ops."""
    E, h, I, G, t = 4, 256, 64, 64, 6
    wl = ms.small_case(3, t, h, I, E, E, G, centred=True)
    r = orc.block(wl)
    lg = torch.from_numpy(orc.router_logits(wl.x, wl.w_router).astype(np.float64))
    p = torch.softmax(lg, dim=1).numpy()
    ref = torch_swiglu(orc, wl.shared_record, h, I, G, xf(wl.x))
    for e in range(E):
        ref = ref + p[:, e:e + 1] * torch_swiglu(orc, wl.records[e], h, I, G, xf(wl.x))
    err = np.max(np.abs(r["out"] - ref))
    assert err <= 1e-6 * np.max(np.abs(ref))


def test_block_without_shared_and_k1(orc):
    """k = 1, no shared expert: each row's output is exactly its single expert's FFN (weight 1)."""
    wl = ms.small_case(4, 20, 256, 64, 5, 1, 64)
    r = orc.block(wl, shared_expert=False)
    assert np.all(r["topk_w"] == 1.0)
    for e in range(5):
        rows = np.nonzero(r["topk_idx"][:, 0] == e)[0]
        if rows.size:
            y = orc.expert_rows(wl.records[e], 256, 64, 64, wl.x, rows)
            assert np.array_equal(r["out"][rows], y.astype(np.float32))


def test_thread_count_does_not_change_bits(tmp_path):
    code = (
        "import sys, numpy as np, moe_synth as ms, oracle\n"
        "wl = ms.small_case(5, 64, 512, 128, 16, 4, 64)\n"
        "r = oracle.block(wl)\n"
        "np.save(sys.argv[1], np.concatenate([r['out'].view(np.uint32).ravel(), r['csr_rows'], r['topk_w'].view(np.uint32).ravel()]))\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for n in (1, 3, 8):
        p = tmp_path / f"o{n}.npy"
        env = dict(os.environ, OMP_NUM_THREADS=str(n), PYTHONPATH=root)
        subprocess.check_call([sys.executable, "-c", code, str(p)], env=env, cwd=root)
        outs.append(np.load(p))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_generator_is_reproducible():
    with open(os.path.join(GOLDEN, "input_hashes.json")) as f:
        want = json.load(f)["hashes"]
    for name in ("tiny", "mid"):
        assert ms.make_workload(name).content_hash() == want[name], name


# ------------------------------------------------------------------ injection into the next norm

def bf16_value(bits):
    return ms.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def test_round_bf16_hand_values(orc):
    """Round to nearest, ties to even, on values placed by hand around 1.0
    (one bf16 ulp there is 2^-7), at the subnormal quantum 2^-133, and past
    the largest finite value."""
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie: to the even neighbour 1.0
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie between 1+2^-7 (odd) and 1+2^-6 (even)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie: up
        (1.0 + 2.0 ** -8 - 2.0 ** -30, 0x3F80),    # just below: down
        (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
        (0.0, 0x0000), (-0.0, 0x8000),
        (2.0 ** -126, 0x0080),                     # smallest normal
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (1.5 * 2.0 ** -133, 0x0002),               # subnormal tie: to even (2 quanta)
        (2.5 * 2.0 ** -133, 0x0002),
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
        (2.0 ** 128, 0x7F80),                      # overflow: infinity
        (3.0, 0x4040), (-0.15625, 0xBE20),
    ]
    got = orc.round_bf16([c[0] for c in cases])
    assert [int(g) for g in got] == [c[1] for c in cases]


def test_round_bf16_equals_generator_on_floats(orc):
    """On values that are exactly float32 a single rounding to bf16 is the
    whole job: equal to the input generator's own float32 -> bf16 rounding."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    assert np.array_equal(orc.round_bf16(v.astype(np.float64)), ms.f32_to_bf16_bits(v))


def test_inject_norm_constant_rows(orc):
    """Rows whose copies are constant give z constant along the row, so with
    eps = 0 the norm is exactly gamma[c] * sign(z): pins the weights alpha
    and beta per copy, the gain's index and the sign."""
    t, n, h = 3, 3, 64
    alpha = np.array([0.5, -0.25, 2.0])
    beta = np.array([1.0, 0.0, -3.0])
    gamma = np.linspace(-2, 2, h).astype(np.float32)
    gamma = bf16_value(bf16(gamma)).astype(np.float32)         # exactly bf16
    cst = np.array([[1.0, 2.0, -1.0], [0.5, 4.0, 0.25], [-1.0, -1.0, -1.0]])   # hyper[r][i]
    yv = np.array([2.0, -1.0, 0.5])
    hyper = np.repeat(cst[:, :, None], h, axis=2).astype(np.float32)
    y = np.repeat(yv[:, None], h, axis=1).astype(np.float32)
    hout, mixed = orc.inject_norm(hyper, y, alpha, beta, gamma, 0.0)
    upd = cst + beta[None, :] * yv[:, None]
    assert np.array_equal(hout, np.repeat(upd[:, :, None], h, axis=2).astype(np.float32))
    z = (alpha[None, :] * upd).sum(axis=1)            # [1.25 - 0 + 2*(-7)...] per row
    assert (z != 0).all()
    want = np.sign(z)[:, None] * gamma[None, :].astype(np.float64)
    assert np.array_equal(bf16_value(mixed), want)


def test_inject_norm_is_residual_plus_rms_norm(orc):
    """One copy with alpha = beta = 1 is the plain pre-norm residual: the next
    block input is torch's float64 rms_norm of hyper + y, correctly rounded
    to bf16 (within half a bf16 ulp of the float64 value)."""
    rng = np.random.default_rng(6)
    t, h = 37, 512
    hyper = rng.standard_normal((t, 1, h)).astype(np.float32)
    y = (0.3 * rng.standard_normal((t, h))).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    eps = 1e-6
    hout, mixed = orc.inject_norm(hyper, y, [1.0], [1.0], gamma, eps)
    z = torch.from_numpy(hyper[:, 0].astype(np.float64)) + torch.from_numpy(y.astype(np.float64))
    ref = torch.nn.functional.rms_norm(z, (h,), weight=torch.from_numpy(gamma.astype(np.float64)), eps=eps).numpy()
    assert np.array_equal(hout[:, 0], (hyper[:, 0].astype(np.float64) + y).astype(np.float32))
    got = bf16_value(mixed)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(ref))) - 7)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-9))


def test_inject_norm_selects_copies(orc):
    """alpha one-hot on copy j reads copy j alone; beta = 0 leaves every copy
    unchanged; y = None injects nothing.  References: torch float64 rms_norm."""
    rng = np.random.default_rng(7)
    t, n, h = 5, 4, 256
    hyper = rng.standard_normal((t, n, h)).astype(np.float32)
    y = rng.standard_normal((t, h)).astype(np.float32)
    gamma = rng.uniform(-1, 1, h).astype(np.float32)
    beta = np.array([0.5, -1.0, 2.0, 0.25], dtype=np.float32)
    for j in range(n):
        alpha = np.eye(n, dtype=np.float32)[j]
        hout, mixed = orc.inject_norm(hyper, y, alpha, beta, gamma, 1e-5)
        z = torch.from_numpy(hyper[:, j].astype(np.float64) + beta[j] * y.astype(np.float64))
        ref = torch.nn.functional.rms_norm(z, (h,), weight=torch.from_numpy(gamma.astype(np.float64)),
                                           eps=1e-5).numpy()
        ulp = 2.0 ** (np.floor(np.log2(np.abs(ref))) - 7)
        assert np.all(np.abs(bf16_value(mixed) - ref) <= 0.5 * ulp * (1 + 1e-9)), j
    hout, _ = orc.inject_norm(hyper, y, np.ones(n), np.zeros(n), gamma, 1e-5)
    assert np.array_equal(hout, hyper)
    hout2, m2 = orc.inject_norm(hyper, None, np.ones(n), beta, gamma, 1e-5)
    assert np.array_equal(hout2, hyper)
    _, m3 = orc.inject_norm(hyper, np.zeros((t, h), np.float32), np.ones(n), beta, gamma, 1e-5)
    assert np.array_equal(m2, m3)


def test_inject_norm_zero_row_with_eps(orc):
    """A row that reads as all zeros normalises to +0 (no NaN) when eps > 0."""
    hyper = np.zeros((2, 2, 64), np.float32)
    hyper[1] = 1.0
    _, mixed = orc.inject_norm(hyper, None, [1.0, -1.0], [0.0, 0.0], np.ones(64, np.float32), 1e-6)
    assert np.all(mixed == 0)


# ------------------------------------------------------------------ low-bit (2-bit) records

def test_layout_2bit_sizes(orc):
    """2-bit records: code sections of h*I/4 bytes, the same scale/bias sections."""
    for h, I, G in [(256, 128, 32), (2048, 768, 64), (4096, 1536, 64)]:
        a = orc.layout(h, I, G, 2)
        b = ms.layout(h, I, G, 2)
        for k, v in a.items():
            assert v == getattr(b, k), (h, I, G, k)
        assert a["gate_sb"] - a["gate_w"] == -(-h * I // 4 // 256) * 256
    assert orc.layout(4096, 1536, 64, 2)["stride"] == 3 * (4096 * 1536 // 4 + 4096 * 1536 // 64 * 4)  # 5,898,240


def test_dequant2_codes_only(orc):
    """scale = 1, bias = 0 -> W = q exactly (pins every 2-bit code position)."""
    h, I, G = 256, 128, 32
    L = ms.layout(h, I, G, 2)
    g = np.random.default_rng(11)
    mats = {}
    for m in ("gate", "up", "down"):
        N, K = ms.matrix_shape(L, m)
        mats[m] = (g.integers(0, 4, (N, K)), np.ones((N, K // G)), np.zeros((N, K // G)))
    rec = ms.pack_record(L, mats, bits=2)
    for m in ("gate", "up", "down"):
        W = orc.dequant(rec, m, h, I, G, bits=2)
        assert np.array_equal(W, mats[m][0].astype(np.float64)), m


def test_dequant2_hand_placed_byte(orc):
    """Byte 2 of word 1 of lane 33 in tile 0 holds the codes of columns
    32 + 16 + {1, 3, 5, 7} of row 1 (lane 33 = row 1, column half 1; byte 2
    = bits 16-23 = the odd codes 1, 3, 5, 7 of the word's 16).  0xE4 puts
    0, 1, 2, 3 there; every other weight is 0."""
    h, I, G = 256, 128, 64
    L = ms.layout(h, I, G, 2)
    rec = np.zeros(L.stride, dtype=np.uint8)
    sb = ms.pack_sb(np.ones((I, h // G)), np.zeros((I, h // G)), G)     # scale 1, bias 0
    rec[L.gate_sb: L.gate_sb + sb.size] = sb
    rec[L.gate_w + 256 * 1 + 4 * 33 + 2] = 0xE4
    W = orc.dequant(rec, "gate", h, I, G, bits=2)
    want = np.zeros((I, h))
    want[1, [49, 51, 53, 55]] = [0, 1, 2, 3]
    assert np.array_equal(W, want)


@pytest.mark.parametrize("centred", [False, True])
def test_2bit_record_equals_4bit_record_with_same_codes(orc, centred):
    """A 2-bit record and a 4-bit record holding the same codes (0..3) and
    scale/bias decode to the same weights, so the block over experts given
    in either form is bitwise the same."""
    h, I, G, E = 256, 128, 32, 6
    wl = ms.small_case(40, 24, h, I, E, 2, G, centred=centred)
    L2 = ms.layout(h, I, G, 2)
    rng = np.random.default_rng(12)
    rec4 = np.zeros_like(wl.records)
    rec2 = np.zeros_like(wl.records)
    for e in range(E):
        mats = {}
        for m in ("gate", "up", "down"):
            N, K = ms.matrix_shape(wl.layout, m)
            s = rng.uniform(0.02, 0.08, (N, K // G)).astype(np.float16)
            b = rng.normal(0, 0.01, (N, K // G)).astype(np.float16)
            if centred:
                b = (b - 1.5 * s).astype(np.float16)
            mats[m] = (rng.integers(0, 4, (N, K)), s, b)
        rec4[e] = ms.pack_record(wl.layout, mats)
        rec2[e, :L2.stride] = ms.pack_record(L2, mats, bits=2)
        for m in ("gate", "up", "down"):
            assert np.array_equal(orc.dequant(rec4[e], m, h, I, G), orc.dequant(rec2[e, :L2.stride], m, h, I, G, 2))
    import dataclasses
    bits = np.array([2, 4, 2, 2, 4, 2], dtype=np.uint8)
    a = orc.block(dataclasses.replace(wl, records=rec4))
    mixed = rec4.copy()
    mixed[bits == 2] = rec2[bits == 2]
    b = orc.block(dataclasses.replace(wl, records=mixed), record_bits=bits)
    assert np.array_equal(a["out"], b["out"])
    s = np.arange(0, 24, 5)
    assert np.array_equal(orc.tokens_bruteforce(dataclasses.replace(wl, records=mixed), s, record_bits=bits),
                          orc.tokens_bruteforce(dataclasses.replace(wl, records=rec4), s))


def test_residency_order_is_stable_sort_by_count(orc):
    """The by-use order equals numpy's stable sort of the non-empty experts
    by descending count (a library routine), and keep marks its first n."""
    rng = np.random.default_rng(21)
    for E in (1, 5, 64, 512, 1024):
        counts = rng.integers(0, 6, E)          # many ties and empty experts
        counts[rng.random(E) < 0.2] = 0
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
        nz = np.nonzero(counts)[0]
        want = nz[np.argsort(-counts[nz], kind="stable")]
        for n_keep in (0, 1, 7, E, E + 3):
            keep, order = orc.residency(offsets, n_keep, with_order=True)
            assert np.array_equal(order[: want.size], want.astype(np.uint32))
            assert (order[want.size:] == 0xFFFFFFFF).all()
            assert np.array_equal(np.nonzero(keep)[0], np.sort(want[:n_keep]))
