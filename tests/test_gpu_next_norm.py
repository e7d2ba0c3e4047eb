"""GPU parity of the next fused norm (the block output injected into the n
residual copies and read back, RMS-normalised, as the next block's input)
through the C ABI: moe_inject_norm on its own, and moe_block_next_norm,
which forms each row's block output in the combine and injects it without
writing it.

Bars:
  - moe_inject_norm against the oracle on the same fp32 inputs: each updated
    copy within one fp32 ulp of the oracle's (the oracle rounds the double
    sum once; the GPU's fma rounds once too, so they differ only where the
    double sum sits on a float tie); each bf16 output within one bf16 ulp of
    the oracle's correctly rounded value plus the fp32 error of the GPU's
    read and norm, (n + 4) 2^-24 sum_i |alpha_i copy_i| |gamma| / rms per
    element (it matters only where the copies nearly cancel), and bitwise
    equal on all but a few elements;
  - moe_block_next_norm bitwise equal to moe_block followed by
    moe_inject_norm on its output (same arithmetic, same order);
  - against the oracle's whole chain (its block output, then its injection
    and norm): with zero expert weights the block output is exactly 0 on
    both sides, so the copies must be unchanged and the norm within one bf16
    ulp; with real weights the injected part and the next input are held to
    the block's bar (relative Frobenius error <= 5e-3, max abs <= 1e-2 max).
"""
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


def bf16_to_f64(bits):
    return ms.bf16_bits_to_f32(np.asarray(bits).view(np.uint16)).astype(np.float64)


def fp32_norm_slack(copies, alpha, gamma, eps):
    """Bound on the GPU's fp32 error before the final rounding, per element:
    (n + 4) u sum_i |alpha_i copy_i| |gamma| / sqrt(mean z^2 + eps), u = 2^-24
    (n fma roundings of the read, then the norm's scale and product)."""
    c = np.asarray(copies, np.float64)
    a = np.asarray(alpha, np.float64)
    n = c.shape[1]
    z = np.einsum("tnh,n->th", c, a)
    rms = np.sqrt(np.mean(z * z, axis=1, keepdims=True) + eps)
    S = np.einsum("tnh,n->th", np.abs(c), np.abs(a))
    return (n + 4) * 2.0 ** -24 * S * np.abs(np.asarray(gamma, np.float64))[None, :] / rms


def within_one_bf16_ulp(got_bits, ref_bits, slack=0.0):
    g, r = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    ulp = np.where(r == 0, 2.0 ** -133, 2.0 ** (np.floor(np.log2(np.abs(np.where(r == 0, 1, r)))) - 7))
    ok = np.abs(g - r) <= ulp + slack
    exact = float(np.mean(np.asarray(got_bits).view(np.uint16) == np.asarray(ref_bits).view(np.uint16)))
    return bool(ok.all()), exact


def within_one_f32_ulp(got, ref):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    up = np.nextafter(ref, np.float32(np.inf))
    dn = np.nextafter(ref, np.float32(-np.inf))
    return bool(((got == ref) | (got == up) | (got == dn)).all()), float(np.mean(got == ref))


def check_rel(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    fro = np.linalg.norm(d) / np.linalg.norm(ref)
    mx = np.max(np.abs(d)) / np.max(np.abs(ref))
    print(f"    {what}: rel_fro={fro:.2e} max_abs_rel={mx:.2e}", flush=True)
    assert fro <= REL_FRO and mx <= MAX_ABS_REL, (what, fro, mx)


def rand_norm_inputs(seed, t, n, h):
    rng = np.random.default_rng(seed)
    hyper = rng.standard_normal((t, n, h)).astype(np.float32)
    y = (0.5 * rng.standard_normal((t, h))).astype(np.float32)
    alpha = rng.uniform(-1, 1, n).astype(np.float32)
    beta = rng.uniform(-2, 2, n).astype(np.float32)
    gamma = rng.uniform(0.25, 2, h).astype(np.float32)
    return hyper, y, alpha, beta, gamma


CASES = [(1, 1, 256), (7, 3, 2048), (300, 4, 4096), (33, 2, 6144), (5, 16, 512), (64, 1, 16384), (4096, 4, 2048)]


@pytest.mark.parametrize("with_y", [True, False], ids=["inject", "read-only"])
@pytest.mark.parametrize("case", CASES, ids=[f"t{c[0]}-n{c[1]}-h{c[2]}" for c in CASES])
def test_inject_norm_against_oracle(mep, orc, case, with_y):
    t, n, h = case
    hyper, y, alpha, beta, gamma = rand_norm_inputs(1000 + t + n + h, t, n, h)
    eps = 1e-6
    d_hyper = torch.from_numpy(hyper).cuda()
    d_y = torch.from_numpy(y).cuda() if with_y else None
    d_gamma = torch.from_numpy(gamma).cuda()
    d_mixed = torch.full((t, h), -1, dtype=torch.int16, device="cuda")
    nn = mep.next_norm(d_hyper, alpha, beta, d_gamma, eps, d_mixed)
    mep.moe_inject_norm(d_y, t, h, nn)
    torch.cuda.synchronize()
    ref_h, ref_m = orc.inject_norm(hyper, y if with_y else None, alpha, beta, gamma, eps)
    ok, exact = within_one_f32_ulp(d_hyper.cpu().numpy(), ref_h)
    assert ok, "updated copies differ from the oracle by more than one fp32 ulp"
    if not with_y:
        assert np.array_equal(d_hyper.cpu().numpy(), hyper)
    okm, exactm = within_one_bf16_ulp(d_mixed.cpu().numpy(), ref_m, fp32_norm_slack(ref_h, alpha, gamma, eps))
    print(f"    copies bitwise {exact:.6f}, next input bitwise {exactm:.6f}", flush=True)
    assert okm, "next block input differs from the oracle by more than one bf16 ulp plus the fp32 bound"
    assert exact > 0.999 and exactm > 0.98


def test_inject_norm_rejects_bad_arguments(mep):
    t, n, h = 4, 2, 256
    hyper = torch.zeros((t, n, h), device="cuda")
    gamma = torch.ones(h, device="cuda")
    mixed = torch.zeros((t, h), dtype=torch.int16, device="cuda")
    with pytest.raises(mep.MoeError):          # h not a multiple of 256
        mep.moe_inject_norm(None, t, 200, mep.next_norm(hyper, [1, 1], [1, 1], gamma, 1e-6, mixed))
    with pytest.raises(mep.MoeError):          # negative eps
        mep.moe_inject_norm(None, t, h, mep.next_norm(hyper, [1, 1], [1, 1], gamma, -1.0, mixed))
    with pytest.raises(mep.MoeError):          # mixed inside hyper
        nn = mep.next_norm(hyper, [1, 1], [1, 1], gamma, 1e-6, mixed)
        nn.mixed = hyper.data_ptr()
        mep.moe_inject_norm(None, t, h, nn)
    with pytest.raises(mep.MoeError):          # empty chunk
        mep.moe_inject_norm(None, 0, h, mep.next_norm(hyper, [1, 1], [1, 1], gamma, 1e-6, mixed))
    torch.cuda.synchronize()
    assert bool((mixed == 0).all())


def block_and_norm(mep, wl, hyper, alpha, beta, gamma, eps, shared=True):
    """Routing outputs, the block's out, and (copies, next input) from
    moe_block + moe_inject_norm, then the same from moe_block_next_norm."""
    t, h = wl.x.shape
    blk = mep.MoeBlock.from_workload(wl, shared=shared)
    d_gamma = torch.from_numpy(gamma).cuda()
    blk.workspace.fill_(0xFF)
    blk.block(accumulate=0)
    out = blk.out.clone()
    h1 = torch.from_numpy(hyper).cuda()
    m1 = torch.full((t, h), -1, dtype=torch.int16, device="cuda")
    mep.moe_inject_norm(out, t, h, mep.next_norm(h1, alpha, beta, d_gamma, eps, m1))
    routing = {k: getattr(blk, k).clone() for k in ("topk_idx", "offsets", "csr_rows", "csr_pos")}
    blk.workspace.fill_(0xFF)
    blk.out.fill_(float("nan"))
    h2 = torch.from_numpy(hyper).cuda()
    m2 = torch.full((t, h), -1, dtype=torch.int16, device="cuda")
    blk.block_next_norm(mep.next_norm(h2, alpha, beta, d_gamma, eps, m2))
    torch.cuda.synchronize()
    for k, v in routing.items():
        assert torch.equal(v, getattr(blk, k)), k
    assert bool(torch.isnan(blk.out).all()), "the fused call must not write out"
    res = dict(out=out.cpu().numpy(), h1=h1.cpu().numpy(), m1=m1.cpu().numpy(), h2=h2.cpu().numpy(),
               m2=m2.cpu().numpy())
    del blk
    return res


WORKLOADS = [("tiny", 3), ("mid", 2), ("decode", 4), ("decode1", 1), ("full", 4)]


@pytest.mark.parametrize("name,n", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_block_next_norm_matches_block_then_norm(mep, orc, name, n):
    """The fused call equals the two calls bitwise; both are held to the
    oracle's chain at the block's bar."""
    wl = ms.make_workload(name, centred=True)
    t, h = wl.x.shape
    hyper, _, alpha, beta, gamma = rand_norm_inputs(77, t, n, h)
    r = block_and_norm(mep, wl, hyper, alpha, beta, gamma, 1e-6)
    assert np.array_equal(r["h1"], r["h2"]), "copies differ between the fused and the separate calls"
    assert np.array_equal(r["m1"], r["m2"]), "next input differs between the fused and the separate calls"
    print(f"  oracle {name} ...", flush=True)
    ref = orc.block(wl, with_logits=False)
    ref_h, ref_m = orc.inject_norm(hyper, ref["out"], alpha, beta, gamma, 1e-6)
    check_rel(r["h2"] - hyper, ref_h.astype(np.float64) - hyper, f"{name} injected part")
    check_rel(bf16_to_f64(r["m2"]), bf16_to_f64(ref_m), f"{name} next input")


def test_block_next_norm_without_shared_expert(mep, orc):
    wl = ms.small_case(31, 130, 512, 128, 24, 4, 64, centred=True)
    hyper, _, alpha, beta, gamma = rand_norm_inputs(78, 130, 2, 512)
    r = block_and_norm(mep, wl, hyper, alpha, beta, gamma, 1e-5, shared=False)
    assert np.array_equal(r["h1"], r["h2"]) and np.array_equal(r["m1"], r["m2"])
    ref = orc.block(wl, shared_expert=False, with_logits=False)
    ref_h, ref_m = orc.inject_norm(hyper, ref["out"], alpha, beta, gamma, 1e-5)
    check_rel(r["h2"] - hyper, ref_h.astype(np.float64) - hyper, "no shared: injected part")
    check_rel(bf16_to_f64(r["m2"]), bf16_to_f64(ref_m), "no shared: next input")


@pytest.mark.parametrize("name", ["mid", "decode"])
def test_block_next_norm_zero_experts(mep, orc, name):
    """All expert weights zero: the block output is exactly zero on both
    sides, so the copies come back unchanged bitwise and the next input is
    the norm of the copies alone, within one bf16 ulp of the oracle."""
    wl = ms.make_workload(name)
    wl.records[:] = 0
    wl.shared_record[:] = 0
    t, h = wl.x.shape
    hyper, _, alpha, beta, gamma = rand_norm_inputs(79, t, 3, h)
    r = block_and_norm(mep, wl, hyper, alpha, beta, gamma, 1e-6)
    assert not r["out"].any()
    assert np.array_equal(r["h2"], hyper)
    _, ref_m = orc.inject_norm(hyper, None, alpha, beta, gamma, 1e-6)
    ok, exact = within_one_bf16_ulp(r["m2"], ref_m, fp32_norm_slack(hyper, alpha, gamma, 1e-6))
    print(f"    next input bitwise {exact:.6f}", flush=True)
    assert ok and exact > 0.98


def residual_inputs(seed, t, n, h):
    hyper, y, a_in, b_in, g_in = rand_norm_inputs(seed, t, n, h)
    rng = np.random.default_rng(seed + 1)
    a_out = rng.uniform(-1, 1, n).astype(np.float32)
    b_out = rng.uniform(-2, 2, n).astype(np.float32)
    g_out = rng.uniform(0.25, 2, h).astype(np.float32)
    return hyper, y, (a_in, b_in, g_in), (a_out, b_out, g_out)


ROUTES = [("mid", 2, True), ("decode", 4, True), ("full", 4, False), ("tiny", 1, True)]


@pytest.mark.parametrize("name,n,fused_out", ROUTES, ids=[f"{c[0]}-n{c[1]}-{'next' if c[2] else 'out'}" for c in ROUTES])
def test_block_from_residual_matches_separate_calls(mep, orc, name, n, fused_out):
    """moe_block_from_residual equals moe_inject_norm (the pending attention
    output into the copies, the block input produced) followed by
    moe_block_next_norm (or moe_block), bitwise, with the same residual
    copies described for both norms; its block input is held to the
    oracle's norm like moe_inject_norm."""
    wl = ms.make_workload(name, centred=True)
    t, h = wl.x.shape
    hyper, y, (a_in, b_in, g_in), (a_out, b_out, g_out) = residual_inputs(500 + n, t, n, h)
    blk = mep.MoeBlock.from_workload(wl)
    d_y = torch.from_numpy(y).cuda()
    g_in_d, g_out_d = torch.from_numpy(g_in).cuda(), torch.from_numpy(g_out).cuda()

    def run(one_call):
        copies = torch.from_numpy(hyper).cuda()
        nxt = torch.full((t, h), -1, dtype=torch.int16, device="cuda")
        blk.x.fill_(float("nan"))
        blk.workspace.fill_(0xFF)
        blk.out.fill_(float("nan"))
        in_nn = mep.next_norm(copies, a_in, b_in, g_in_d, 1e-6, blk.x)
        out_nn = mep.next_norm(copies, a_out, b_out, g_out_d, 1e-6, nxt) if fused_out else None
        if one_call:
            mep.moe_block_from_residual(d_y, in_nn, blk.w_router, t, blk.k, blk.L, blk.table, blk.Ls,
                                        blk.shared_record, blk.gate_w, blk.logits, blk.topk_idx, blk.topk_w,
                                        blk.offsets, blk.csr_rows, blk.csr_w, blk.csr_pos, out_nn,
                                        None if fused_out else blk.out, 0, blk.workspace)
        else:
            mep.moe_inject_norm(d_y, t, h, in_nn)
            if fused_out:
                blk.block_next_norm(out_nn)
            else:
                blk.block(accumulate=0)
        torch.cuda.synchronize()
        res = dict(copies=copies.cpu().numpy(), x=blk.x.view(torch.int16).cpu().numpy(), nxt=nxt.cpu().numpy(),
                   out=blk.out.cpu().numpy(), idx=blk.topk_idx.cpu().numpy(), rows=blk.csr_rows.cpu().numpy())
        return res

    a = run(False)
    b = run(True)
    for key in ("copies", "x", "nxt", "idx", "rows"):
        assert np.array_equal(a[key], b[key]), key
    if not fused_out:
        assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
        assert np.isfinite(b["out"]).all()
    # the block input against the oracle's injection and norm
    ref_h, ref_x = orc.inject_norm(hyper, y, a_in, b_in, g_in, 1e-6)
    ok, exact = within_one_bf16_ulp(b["x"], ref_x, fp32_norm_slack(ref_h, a_in, g_in, 1e-6))
    print(f"    block input bitwise {exact:.6f}", flush=True)
    assert ok and exact > 0.98
    del blk
