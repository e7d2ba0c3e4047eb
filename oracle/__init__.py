"""ctypes wrapper of the plain CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module.  The GPU package never imports it, and it
imports nothing from the GPU package.  Inputs come from ``moe_synth``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        _lib.orc_layout.argtypes = [I, I, I, P]
        _lib.orc_dequant.argtypes = [P, P, I, I, I, P]
        _lib.orc_router_logits.argtypes = [P, P, I, I, I, P]
        _lib.orc_topk.argtypes = [P, I, I, I, P, P]
        _lib.orc_build_csr.argtypes = [P, P, I, I, I, P, P, P, P]
        _lib.orc_residency.argtypes = [P, I, I, P]
        _lib.orc_residency_order.argtypes = [P, I, I, P, P]
        _lib.orc_expert_rows.argtypes = [P, I, I, I, P, P, I, P]
        _lib.orc_shared.argtypes = [P, I, I, I, P, I, P, P]
        _lib.orc_layout_bits.argtypes = [I, I, I, I, P]
        _lib.orc_dequant2.argtypes = [P, P, I, I, I, P]
        _lib.orc_block.argtypes = [P, P, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
        _lib.orc_tokens_bruteforce.argtypes = [P, P, I, I, I, I, I, I, I, P, P, P, P, P, I, I, P]
        _lib.orc_round_bf16.argtypes = [ctypes.c_double]
        _lib.orc_round_bf16.restype = ctypes.c_uint16
        _lib.orc_inject_norm.argtypes = [P, P, I, I, I, P, P, P, ctypes.c_double, P, P]
        _lib.orc_inject_norm.restype = ctypes.c_int
        _lib.orc_set_threads.argtypes = [I]
        _lib.orc_set_threads.restype = None
        for f in ("orc_layout", "orc_layout_bits", "orc_router_logits", "orc_topk", "orc_build_csr", "orc_expert_rows",
                  "orc_shared", "orc_block", "orc_tokens_bruteforce", "orc_max_threads"):
            getattr(_lib, f).restype = ctypes.c_int
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid input")


def max_threads() -> int:
    return lib().orc_max_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops; every output belongs to one
    thread, so results are bitwise the same at any count."""
    lib().orc_set_threads(int(n))


def layout(hidden: int, inter: int, group: int, bits: int = 4) -> dict:
    out = np.zeros(7, dtype=np.uint64)
    _check(lib().orc_layout_bits(hidden, inter, group, bits, _p(out)), "layout")
    keys = ["gate_w", "gate_sb", "up_w", "up_sb", "down_w", "down_sb", "stride"]
    return {k: int(v) for k, v in zip(keys, out)}


def dequant(record: np.ndarray, matrix: str, hidden: int, inter: int, group: int, bits: int = 4) -> np.ndarray:
    """Decode matrix 'gate' | 'up' | 'down' of one record (4- or 2-bit codes) to float64 [N, K]."""
    L = layout(hidden, inter, group, bits)
    N, K = (inter, hidden) if matrix in ("gate", "up") else (hidden, inter)
    rec = np.ascontiguousarray(record, dtype=np.uint8)
    W = np.empty((N, K), dtype=np.float64)
    base = rec.ctypes.data
    f = lib().orc_dequant if bits == 4 else lib().orc_dequant2
    f(base + L[matrix + "_w"], base + L[matrix + "_sb"], N, K, group, _p(W))
    return W


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w_router, dtype=np.float32)
    t, h = x.shape
    E = w.shape[0]
    out = np.empty((t, E), dtype=np.float32)
    _check(lib().orc_router_logits(_p(x), _p(w), t, h, E, _p(out)), "router_logits")
    return out


def topk(logits: np.ndarray, k: int):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    t, E = lg.shape
    idx = np.empty((t, k), dtype=np.uint32)
    w = np.empty((t, k), dtype=np.float32)
    _check(lib().orc_topk(_p(lg), t, E, k, _p(idx), _p(w)), "topk")
    return idx, w


def build_csr(idx: np.ndarray, wts: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    wts = np.ascontiguousarray(wts, dtype=np.float32)
    t, k = idx.shape
    offsets = np.empty(E + 1, dtype=np.uint32)
    rows = np.empty(t * k, dtype=np.uint32)
    cw = np.empty(t * k, dtype=np.float32)
    pos = np.empty(t * k, dtype=np.uint32)
    _check(lib().orc_build_csr(_p(idx), _p(wts), t, k, E, _p(offsets), _p(rows), _p(cw), _p(pos)), "build_csr")
    return offsets, rows, cw, pos


def residency(offsets: np.ndarray, n_keep: int, with_order: bool = False):
    """keep[e] (bool) for the first n_keep non-empty experts by descending
    rows (stable in id); with_order also returns that order (u32, 0xFFFFFFFF
    past the last non-empty expert)."""
    offsets = np.ascontiguousarray(offsets, dtype=np.uint32)
    E = offsets.size - 1
    keep = np.empty(E, dtype=np.uint8)
    order = np.empty(E, dtype=np.uint32)
    lib().orc_residency_order(_p(offsets), E, n_keep, _p(keep), _p(order))
    return (keep.astype(bool), order) if with_order else keep.astype(bool)


def expert_rows(record: np.ndarray, hidden: int, inter: int, group: int, x: np.ndarray,
                rows: Sequence[int]) -> np.ndarray:
    rec = np.ascontiguousarray(record, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    r = np.ascontiguousarray(rows, dtype=np.uint32)
    y = np.empty((r.size, hidden), dtype=np.float64)
    _check(lib().orc_expert_rows(_p(rec), hidden, inter, group, _p(x), _p(r), r.size, _p(y)), "expert_rows")
    return y


def shared(record: np.ndarray, hidden: int, inter: int, group: int, x: np.ndarray,
           gate_w: Optional[np.ndarray] = None) -> np.ndarray:
    rec = np.ascontiguousarray(record, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    g = None if gate_w is None else np.ascontiguousarray(gate_w, dtype=np.uint16)
    ys = np.empty((x.shape[0], hidden), dtype=np.float64)
    _check(lib().orc_shared(_p(rec), hidden, inter, group, _p(x), x.shape[0], _p(g), _p(ys)), "shared")
    return ys


def _record_ptrs(records: np.ndarray):
    recs = np.ascontiguousarray(records, dtype=np.uint8)
    ptrs = (ctypes.c_void_p * recs.shape[0])(*[recs.ctypes.data + e * recs.shape[1] for e in range(recs.shape[0])])
    return recs, ptrs


def _bits_arg(record_bits):
    return None if record_bits is None else np.ascontiguousarray(record_bits, dtype=np.uint8)


def block(wl, shared_expert: bool = True, with_logits: bool = True, record_bits=None):
    """Whole block through the grouped path. Returns dict of outputs (and the
    router logits in the fixed fp32 order, unless with_logits is False).
    record_bits[e] (4 or 2) gives the code width of expert e's record in
    wl.records (a 2-bit record occupies the start of its row); None: all 4."""
    c = wl.cfg
    x = np.ascontiguousarray(wl.x, dtype=np.uint16)
    t = x.shape[0]
    recs, ptrs = _record_ptrs(wl.records)
    rb = _bits_arg(record_bits)
    out = np.empty((t, c.hidden), dtype=np.float32)
    idx = np.empty((t, c.k), dtype=np.uint32)
    w = np.empty((t, c.k), dtype=np.float32)
    offsets = np.empty(c.experts + 1, dtype=np.uint32)
    rows = np.empty(t * c.k, dtype=np.uint32)
    cw = np.empty(t * c.k, dtype=np.float32)
    pos = np.empty(t * c.k, dtype=np.uint32)
    srec = np.ascontiguousarray(wl.shared_record) if shared_expert else None
    gate = None if wl.gate_w is None else np.ascontiguousarray(wl.gate_w, dtype=np.uint16)
    wr = np.ascontiguousarray(wl.w_router, dtype=np.float32)
    _check(lib().orc_block(_p(x), _p(wr), t, c.hidden, c.inter, c.inter_shared, c.experts, c.k, c.group,
                           ptrs, _p(rb), _p(srec), _p(gate), _p(out), _p(idx), _p(w), _p(offsets), _p(rows),
                           _p(cw), _p(pos)), "block")
    res = dict(out=out, topk_idx=idx, topk_w=w, offsets=offsets, csr_rows=rows, csr_w=cw, csr_pos=pos)
    if with_logits:
        res["logits"] = router_logits(x, wr)
    return res


def round_bf16(values) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of doubles, rounded to nearest, ties to even."""
    v = np.asarray(values, dtype=np.float64)
    f = lib().orc_round_bf16
    return np.array([f(float(a)) for a in v.reshape(-1)], dtype=np.uint16).reshape(v.shape)


def inject_norm(hyper: np.ndarray, y: Optional[np.ndarray], alpha, beta, gamma, eps: float):
    """The block output y [t, h] injected into the n residual copies hyper
    [t, n, h] with weights beta, read back with weights alpha, RMS-normalised
    with gain gamma [h]: returns (updated hyper fp32 [t, n, h], next block
    input as bf16 bit patterns [t, h])."""
    hy = np.ascontiguousarray(hyper, dtype=np.float32)
    t, n, h = hy.shape
    yy = None if y is None else np.ascontiguousarray(y, dtype=np.float32)
    if yy is not None:
        assert yy.shape == (t, h)
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    b = np.ascontiguousarray(beta, dtype=np.float32)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    assert a.shape == (n,) and b.shape == (n,) and g.shape == (h,)
    hout = np.empty_like(hy)
    mixed = np.empty((t, h), dtype=np.uint16)
    _check(lib().orc_inject_norm(_p(hy), _p(yy), t, n, h, _p(a), _p(b), _p(g), float(eps), _p(hout), _p(mixed)),
           "inject_norm")
    return hout, mixed


def tokens_bruteforce(wl, sample: Sequence[int], order: int = 0, shared_expert: bool = True,
                      record_bits=None) -> np.ndarray:
    """Per-token outputs (float64) of the sample rows, computed without grouping."""
    c = wl.cfg
    rb = _bits_arg(record_bits)
    x = np.ascontiguousarray(wl.x, dtype=np.uint16)
    recs, ptrs = _record_ptrs(wl.records)
    s = np.ascontiguousarray(sample, dtype=np.int32)
    out = np.empty((s.size, c.hidden), dtype=np.float64)
    srec = np.ascontiguousarray(wl.shared_record) if shared_expert else None
    gate = None if wl.gate_w is None else np.ascontiguousarray(wl.gate_w, dtype=np.uint16)
    wr = np.ascontiguousarray(wl.w_router, dtype=np.float32)
    _check(lib().orc_tokens_bruteforce(_p(x), _p(wr), x.shape[0], c.hidden, c.inter, c.inter_shared,
                                       c.experts, c.k, c.group, ptrs, _p(rb), _p(srec), _p(gate), _p(s), s.size,
                                       order, _p(out)), "tokens_bruteforce")
    return out
