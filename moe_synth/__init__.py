"""Seeded synthetic inputs for the routed-expert MoE prefill block.

This module only *makes inputs*: it draws seeded random tensors and encodes
them into the byte formats the block consumes (bf16 activations, fp32 router
weights, 4-bit expert records).  It holds none of the block's arithmetic (no
dot products, no routing, no softmax, no grouping) and imports neither the
oracle nor the GPU package; both of those consume the buffers made here.

Workload shapes follow the prefill design described on the cherenkov
``prefill.rs`` source page (module doc: a prompt chunk of up to a few thousand
rows, ``MAX_PREFILL_ROWS`` = 4096) and the expert-record structure on the
``prefill/experts.rs`` page (``pf_experts``: gate/up matrices are inter x
hidden, down is hidden x inter, each stored as 4-bit codes with a per-group
scale and bias).

Record format (the stored layout, moved verbatim by the expert ring):

* Matrices in order gate [I x h], up [I x h], down [h x I] (rows = outputs,
  columns = inputs; groups of ``G`` run along the input dimension).
* Each matrix has a code section and a scale/bias ("sb") section.  Sections
  are laid back to back in the order gate codes, gate sb, up codes, up sb,
  down codes, down sb, each padded to 256 bytes; the record stride is padded
  to 4096 bytes.
* Code section: the matrix is cut into tiles of 32 rows x 64 columns, tile
  (ob, kb) at byte ``(ob * (K/64) + kb) * 1024``.  Inside a tile, "lane"
  ``L`` in [0, 64) owns 16 bytes at ``16 * L``: row ``32*ob + L % 32``,
  columns ``64*kb + 32*(L // 32) + c`` for c in [0, 32).  Code c sits in the
  little-endian 32-bit word ``c // 8`` of those 16 bytes, at bit
  ``4 * ((c % 8) // 2) + 16 * (c % 2)``.
* SB section: per tile in the same order, ``(64/G) * 32`` entries of 4 bytes,
  entry ``gi * 32 + (row % 32)`` for group ``gi`` inside the tile; each entry
  is (scale fp16, bias fp16), little-endian, scale first.
* Weight value: ``W[n, k] = scale * q + bias`` for the group ``k // G``,
  with the code ``q`` unsigned in 0..15.

Low-bit (2-bit) records, the form in which streamed experts may cross the
host link: the same sections in the same order with the same scale/bias
layout; codes are unsigned 0..3 and a code tile (32 rows x 64 columns) is
512 bytes, tile (ob, kb) at ``(ob * (K/64) + kb) * 512``.  Lane ``L`` (row
``32*ob + L % 32``, columns ``64*kb + 32*(L // 32) + c``, c in [0, 32)) owns
two little-endian 32-bit words, word ``j`` at byte ``256 * j + 4 * L`` of
the tile; code c sits in word ``c // 16`` at bit
``2 * ((c % 16) // 2) + 16 * (c % 2)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import json
import os
import zlib
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

SEED = 0
ROUTER_STD = 0.02
SCALE_LO, SCALE_HI = 0.005, 0.02
BIAS_STD = 0.01
TILE_ROWS, TILE_COLS, TILE_BYTES = 32, 64, 1024
SECTION_ALIGN, STRIDE_ALIGN = 256, 4096

_HERE = os.path.dirname(os.path.abspath(__file__))


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic MoE-layer workload."""

    name: str
    t: int            # token rows in the chunk
    hidden: int       # h
    inter: int        # I, routed expert intermediate size
    inter_shared: int  # I_s, shared expert intermediate size
    experts: int      # E
    k: int            # experts per token
    group: int        # G, quantisation group along the input dimension
    zipf_s: float = 0.0    # target Zipf exponent of expert popularity (0 = plain router)
    resident: int = 0      # experts kept in HBM when the rest stream (0 = all resident)
    description: str = ""


CONFIGS: Dict[str, Config] = {
    c.name: c
    for c in [
        Config("tiny", 16, 256, 128, 128, 8, 2, 32,
               description="tiny MoE layer, all experts resident"),
        Config("decode", 8, 4096, 1536, 1536, 512, 10, 64,
               description="decode-shaped weight-streaming case, t=8"),
        Config("decode1", 1, 4096, 1536, 1536, 512, 10, 64,
               description="decode-shaped weight-streaming case, t=1"),
        Config("mid", 512, 2048, 768, 768, 64, 8, 64,
               description="mid prefill chunk, uniform-ish routing"),
        Config("full", 4096, 2048, 768, 768, 128, 8, 64, zipf_s=1.1,
               description="full prefill chunk, Zipf(1.1) expert popularity"),
        Config("large", 4096, 4096, 1536, 1536, 512, 10, 64, zipf_s=1.0, resident=64,
               description="large-model chunk, Zipf(1.0), top-64 experts resident, rest streamed"),
    ]
}


def _zipf_alpha() -> Dict[str, float]:
    path = os.path.join(_HERE, "zipf_alpha.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return {k: float(v["alpha"]) for k, v in json.load(f).items()}


# ---------------------------------------------------------------- random streams

def rng(cfg_name: str, tensor: str, index: int = 0, seed: int = SEED) -> np.random.Generator:
    """Independent PCG64 stream keyed by (seed, config, tensor name, index)."""
    key = [seed, zlib.crc32(cfg_name.encode()), zlib.crc32(tensor.encode()), index]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- record format

@dataclasses.dataclass(frozen=True)
class Layout:
    """Byte offsets of the six sections of one expert record."""

    hidden: int
    inter: int
    group: int
    gate_w: int
    gate_sb: int
    up_w: int
    up_sb: int
    down_w: int
    down_sb: int
    stride: int

    def section(self, name: str) -> int:
        return getattr(self, name)


def _align(n: int, a: int) -> int:
    return (n + a - 1) // a * a


def layout(hidden: int, inter: int, group: int, bits: int = 4) -> Layout:
    """Section offsets of the record format stated in this module's docstring."""
    assert group in (32, 64), "group must be 32 or 64"
    assert bits in (2, 4), "codes of 4 or 2 bits"
    assert hidden % 64 == 0 and inter % 64 == 0, "hidden and inter must be multiples of 64"
    codes = hidden * inter * bits // 8
    sb = hidden * inter // group * 4
    off = 0
    out = {}
    for m in ("gate", "up", "down"):
        out[m + "_w"] = off
        off = _align(off + codes, SECTION_ALIGN)
        out[m + "_sb"] = off
        off = _align(off + sb, SECTION_ALIGN)
    return Layout(hidden, inter, group, stride=_align(off, STRIDE_ALIGN), **out)


def matrix_shape(L: Layout, m: str):
    """(rows, cols) = (outputs, inputs) of matrix m in {'gate','up','down'}."""
    return (L.inter, L.hidden) if m in ("gate", "up") else (L.hidden, L.inter)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Encode codes q[N, K] (values 0..15) into the tiled code section bytes."""
    N, K = q.shape
    assert N % TILE_ROWS == 0 and K % TILE_COLS == 0
    q = np.asarray(q, dtype=np.uint32)
    assert q.max(initial=0) < 16
    # n = 32*ob + r ; k = 64*kb + 32*half + 8*dw + j
    v = q.reshape(N // 32, 32, K // 64, 2, 4, 8)
    j = np.arange(8)
    shift = (4 * (j // 2) + 16 * (j % 2)).astype(np.uint32)
    words = (v << shift).sum(axis=-1, dtype=np.uint32)          # [ob, r, kb, half, dw]
    words = words.transpose(0, 2, 3, 1, 4)                        # [ob, kb, half, r, dw]
    return np.ascontiguousarray(words).astype("<u4").view(np.uint8).reshape(-1)


def pack_codes2(q: np.ndarray) -> np.ndarray:
    """Encode codes q[N, K] (values 0..3) into the tiled 2-bit code section bytes."""
    N, K = q.shape
    assert N % TILE_ROWS == 0 and K % TILE_COLS == 0
    q = np.asarray(q, dtype=np.uint32)
    assert q.max(initial=0) < 4
    # n = 32*ob + r ; k = 64*kb + 32*half + 16*j + c16, c16 = 2*u + odd
    v = q.reshape(N // 32, 32, K // 64, 2, 2, 16)                 # [ob, r, kb, half, j, c16]
    c16 = np.arange(16)
    shift = (2 * (c16 // 2) + 16 * (c16 % 2)).astype(np.uint32)
    words = (v << shift).sum(axis=-1, dtype=np.uint32)            # [ob, r, kb, half, j]
    words = words.transpose(0, 2, 4, 3, 1)                         # [ob, kb, j, half, r] -> lane = 32*half + r
    return np.ascontiguousarray(words).astype("<u4").view(np.uint8).reshape(-1)


def pack_sb(scale: np.ndarray, bias: np.ndarray, group: int) -> np.ndarray:
    """Encode fp16 scale/bias [N, K/G] into the tiled sb section bytes."""
    N, ng = scale.shape
    per_tile = 64 // group
    K = ng * group
    s = np.asarray(scale, dtype=np.float16).view(np.uint16).astype(np.uint32)
    b = np.asarray(bias, dtype=np.float16).view(np.uint16).astype(np.uint32)
    e = s | (b << 16)                                              # [N, K/G]
    e = e.reshape(N // 32, 32, K // 64, per_tile).transpose(0, 2, 3, 1)  # [ob, kb, gi, r]
    return np.ascontiguousarray(e).astype("<u4").view(np.uint8).reshape(-1)


def pack_record(L: Layout, mats: Dict[str, tuple], bits: int = 4) -> np.ndarray:
    """Build one record from logical matrices: mats[m] = (q[N,K], scale[N,K/G], bias[N,K/G])."""
    rec = np.zeros(L.stride, dtype=np.uint8)
    for m in ("gate", "up", "down"):
        q, s, b = mats[m]
        assert q.shape == matrix_shape(L, m)
        cw = pack_codes(q) if bits == 4 else pack_codes2(q)
        sb = pack_sb(s, b, L.group)
        rec[L.section(m + "_w"): L.section(m + "_w") + cw.size] = cw
        rec[L.section(m + "_sb"): L.section(m + "_sb") + sb.size] = sb
    return rec


def random_record(L: Layout, g: np.random.Generator, centred: bool = False, bits: int = 4) -> np.ndarray:
    """One record with uniform codes, scale ~ U(0.005, 0.02) and bias ~ N(0, 0.01^2), as fp16.

    Codes are uniform random bytes, so their order inside the section does not
    matter.  ``centred`` draws bias = -7.5*scale + N(0, 0.01^2) so that weights
    are roughly zero-mean.  With ``bits`` = 2 the codes span 0..3, so the
    scale is drawn 5 times larger (the weights then span the same range) and
    the centred bias is -1.5*scale + N(0, 0.01^2).
    """
    rec = np.zeros(L.stride, dtype=np.uint8)
    qmax = (1 << bits) - 1
    for m in ("gate", "up", "down"):
        N, K = matrix_shape(L, m)
        nb = N * K * bits // 8
        rec[L.section(m + "_w"): L.section(m + "_w") + nb] = np.frombuffer(g.bytes(nb), dtype=np.uint8)
        ne = N * K // L.group
        s = g.uniform(SCALE_LO, SCALE_HI, ne) * (15 / qmax)
        b = g.normal(0.0, BIAS_STD, ne)
        if centred:
            b = b - qmax / 2 * s.astype(np.float16).astype(np.float64)
        s16 = s.astype(np.float16).view(np.uint16).astype(np.uint32)
        b16 = b.astype(np.float16).view(np.uint16).astype(np.uint32)
        e = (s16 | (b16 << 16)).astype("<u4").view(np.uint8)
        rec[L.section(m + "_sb"): L.section(m + "_sb") + e.size] = e
    return rec


# ---------------------------------------------------------------- workload tensors

@dataclasses.dataclass
class Workload:
    cfg: Config
    x: np.ndarray          # uint16 bf16 bits [t, h]
    w_router: np.ndarray   # float32 [E, h]
    layout: Layout         # routed expert record layout
    records: np.ndarray    # uint8 [E, stride]
    shared_layout: Layout
    shared_record: np.ndarray  # uint8 [stride_s]
    gate_w: Optional[np.ndarray] = None  # uint16 bf16 bits [h] or None

    def content_hash(self) -> str:
        h = hashlib.sha256()
        for a in (self.x, self.w_router, self.records, self.shared_record):
            h.update(np.ascontiguousarray(a).view(np.uint8).data)
        if self.gate_w is not None:
            h.update(self.gate_w.view(np.uint8).data)
        return h.hexdigest()[:16]


def make_x(cfg: Config, t: Optional[int] = None) -> np.ndarray:
    t = cfg.t if t is None else t
    return f32_to_bf16_bits(rng(cfg.name, "x").standard_normal((t, cfg.hidden), dtype=np.float32))


def zipf_gain(cfg: Config, alpha: Optional[float] = None) -> np.ndarray:
    """Per-expert row gain (pi(e)+1)^-alpha that skews routing towards Zipf popularity."""
    if alpha is None:
        alpha = _zipf_alpha().get(cfg.name, 0.0) if cfg.zipf_s else 0.0
    perm = rng(cfg.name, "zipf_perm").permutation(cfg.experts)
    return (perm + 1.0) ** (-alpha)


def make_router(cfg: Config, alpha: Optional[float] = None) -> np.ndarray:
    w = rng(cfg.name, "w_router").normal(0.0, ROUTER_STD, (cfg.experts, cfg.hidden))
    if cfg.zipf_s:
        w = w * zipf_gain(cfg, alpha)[:, None]
    return w.astype(np.float32)


def make_records(cfg: Config, experts: Optional[Iterable[int]] = None, centred: bool = False,
                 bits: int = 4) -> np.ndarray:
    """Records [n, stride] for the given experts (default: all E), each from its own stream."""
    L = layout(cfg.hidden, cfg.inter, cfg.group, bits)
    ids = list(range(cfg.experts)) if experts is None else list(experts)
    out = np.empty((len(ids), L.stride), dtype=np.uint8)
    tag = ("record_c" if centred else "record") + ("" if bits == 4 else f"_b{bits}")
    for i, e in enumerate(ids):
        out[i] = random_record(L, rng(cfg.name, tag, e), centred, bits)
    return out


def make_shared(cfg: Config, centred: bool = False) -> np.ndarray:
    L = layout(cfg.hidden, cfg.inter_shared, cfg.group)
    return random_record(L, rng(cfg.name, "shared_c" if centred else "shared"), centred)


def make_gate(cfg: Config) -> np.ndarray:
    return f32_to_bf16_bits(rng(cfg.name, "gate_w").normal(0.0, ROUTER_STD, cfg.hidden).astype(np.float32))


def make_workload(cfg, centred: bool = False, with_gate: bool = False, t: Optional[int] = None) -> Workload:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return Workload(
        cfg=cfg,
        x=make_x(cfg, t),
        w_router=make_router(cfg),
        layout=layout(cfg.hidden, cfg.inter, cfg.group),
        records=make_records(cfg, centred=centred),
        shared_layout=layout(cfg.hidden, cfg.inter_shared, cfg.group),
        shared_record=make_shared(cfg, centred),
        gate_w=make_gate(cfg) if with_gate else None,
    )


def small_case(seed: int, t: int, hidden: int, inter: int, experts: int, k: int, group: int,
               inter_shared: Optional[int] = None, centred: bool = False, with_gate: bool = False) -> Workload:
    """A random small workload for property and parity sweeps."""
    name = f"small-{seed}-{t}-{hidden}-{inter}-{experts}-{k}-{group}"
    cfg = Config(name, t, hidden, inter, inter_shared or inter, experts, k, group)
    return make_workload(cfg, centred=centred, with_gate=with_gate)
