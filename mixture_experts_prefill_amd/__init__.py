"""Routed-expert MoE prefill block on MI355X: Python binding of libmoe.

Thin ctypes marshalling over the C ABI in ``include/moe.h``: every function
here has the name of the C entry point it calls, takes torch tensors that
already live on the GPU, passes their device pointers and the current HIP
stream, and raises ``MoeError`` on a non-zero status.  All computation runs
in the HIP kernels of ``libmoe.so``; nothing here computes on the host.
The library must be built first (``python -m mixture_experts_prefill_amd.build``);
importing the functions without it raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH names another build of the same library (for side-by-side timing)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_HERE, "libmoe.so")
MAX_ROWS = 4096
MAX_EXPERTS = 1024
MAX_K = 32

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID", 2: "MOE_ERR_CAPACITY", 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class moe_layout(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("group", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("gate_w", ctypes.c_uint64), ("gate_sb", ctypes.c_uint64),
                ("up_w", ctypes.c_uint64), ("up_sb", ctypes.c_uint64), ("down_w", ctypes.c_uint64),
                ("down_sb", ctypes.c_uint64), ("stride", ctypes.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


MAX_HC = 16   # MOE_MAX_HC of include/moe.h


class moe_next_norm(ctypes.Structure):
    _fields_ = [("hyper", ctypes.c_void_p), ("n", ctypes.c_int32), ("alpha", ctypes.c_float * MAX_HC),
                ("beta", ctypes.c_float * MAX_HC), ("gamma", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("mixed", ctypes.c_void_p)]


class moe_ring_stats(ctypes.Structure):
    _fields_ = [("jobs", ctypes.c_int32), ("streamed", ctypes.c_int32), ("batches", ctypes.c_int32),
                ("fetched_bytes", ctypes.c_uint64), ("wait_ms", ctypes.c_double)]


_lib = None
EXPORTS = ["moe_last_error", "moe_layout_make", "moe_workspace_bytes", "moe_route", "moe_build_csr",
           "moe_shared", "moe_ring_create", "moe_ring_destroy", "moe_ring_get_stats", "moe_prefill_experts",
           "moe_ring_plan_debug", "moe_profile_begin", "moe_profile_end", "moe_profile_set_mask",
           "moe_prefill_fused", "moe_block", "moe_block_noalloc", "moe_inject_norm", "moe_block_next_norm",
           "moe_layout_make_bits", "moe_ring_set_miss_layout", "moe_residency", "moe_lookahead",
           "moe_block_from_residual", "moe_chunk_stats_fill", "moe_debug_read_probe",
           "moe_debug_schedule", "moe_debug_xcc_map", "moe_debug_tile_wait"]
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h
PHASES = ["router", "topk", "csr", "shared_gateup", "shared_down", "schedule", "gateup", "down", "combine", "norm",
          "experts"]


def lib():
    """Load libmoe.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run python -m mixture_experts_prefill_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP = ctypes.POINTER(moe_layout)
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_layout_make.argtypes = [I, I, I, LP]
    L.moe_layout_make_bits.argtypes = [I, I, I, I, LP]
    L.moe_ring_set_miss_layout.argtypes = [P, LP, P]
    L.moe_workspace_bytes.argtypes = [I, I, I, LP, LP]
    L.moe_workspace_bytes.restype = Z
    L.moe_route.argtypes = [P, P, I, I, I, I, P, P, P, P]
    L.moe_build_csr.argtypes = [P, P, I, I, I, P, P, P, P, P, Z, P]
    L.moe_shared.argtypes = [P, I, LP, P, P, P, I, P, Z, P]
    L.moe_ring_create.argtypes = [LP, P, I, I, ctypes.POINTER(P)]
    L.moe_ring_destroy.argtypes = [P]
    L.moe_ring_destroy.restype = None
    L.moe_ring_get_stats.argtypes = [P, ctypes.POINTER(moe_ring_stats)]
    L.moe_prefill_experts.argtypes = [P, I, I, I, LP, P, P, P, P, P, P, P, P, I, P, Z, P]
    L.moe_prefill_fused.argtypes = [P, I, I, I, LP, P, P, P, P, P, LP, P, P, P, I, P, Z, P]
    L.moe_block.argtypes = [P, P, I, I, I, LP, P, LP, P, P, P, P, P, P, P, P, P, P, I, P, Z, P]
    L.moe_block_noalloc.argtypes = [P, P, I, I, I, LP, P, LP, P, P, P, P, P, P, P, P, P, P, I, P]
    NP = ctypes.POINTER(moe_next_norm)
    L.moe_inject_norm.argtypes = [P, I, I, NP, P]
    L.moe_block_next_norm.argtypes = [P, P, I, I, I, LP, P, LP, P, P, P, P, P, P, P, P, P, NP, P, Z, P]
    L.moe_residency.argtypes = [P, I, I, P, P, P]
    L.moe_chunk_stats_fill.argtypes = [P, I, I, P, P]
    L.moe_debug_read_probe.argtypes = [P, Z, I, P, P]
    L.moe_debug_read_probe.restype = ctypes.c_int
    L.moe_debug_schedule.argtypes = [P, I, I, I, P, P, I, I, P, P, I, P]
    L.moe_debug_schedule.restype = ctypes.c_int
    L.moe_debug_xcc_map.argtypes = [P, I, P]
    L.moe_debug_xcc_map.restype = ctypes.c_int
    L.moe_debug_tile_wait.argtypes = [I, I]
    L.moe_debug_tile_wait.restype = ctypes.c_int
    L.moe_lookahead.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P, P]
    L.moe_block_from_residual.argtypes = [P, NP, P, I, I, I, LP, P, LP, P, P, P, P, P, P, P, P, P, NP, P, I, P, Z,
                                          P]
    L.moe_ring_plan_debug.argtypes = [P, P, I, I, I, P, P, P]
    L.moe_profile_begin.argtypes = [ctypes.c_uint32]
    L.moe_profile_begin.restype = None
    L.moe_profile_set_mask.argtypes = [ctypes.c_uint32]
    L.moe_profile_set_mask.restype = None
    L.moe_profile_end.argtypes = [P, P]
    L.moe_profile_end.restype = ctypes.c_int
    for f in ("moe_layout_make", "moe_layout_make_bits", "moe_ring_set_miss_layout", "moe_route", "moe_build_csr", "moe_shared", "moe_ring_create",
              "moe_ring_get_stats", "moe_prefill_experts", "moe_prefill_fused", "moe_block", "moe_block_noalloc", "moe_inject_norm", "moe_block_next_norm",
              "moe_residency", "moe_lookahead", "moe_block_from_residual", "moe_chunk_stats_fill"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ------------------------------------------------------------------ entry points

def moe_layout_make(hidden: int, inter: int, group: int) -> moe_layout:
    out = moe_layout()
    _check(lib().moe_layout_make(hidden, inter, group, ctypes.byref(out)))
    return out


def moe_layout_make_bits(hidden: int, inter: int, group: int, bits: int) -> moe_layout:
    out = moe_layout()
    _check(lib().moe_layout_make_bits(hidden, inter, group, bits, ctypes.byref(out)))
    return out


def moe_workspace_bytes(t: int, k: int, E: int, routed: moe_layout, shared: Optional[moe_layout] = None) -> int:
    return lib().moe_workspace_bytes(t, k, E, ctypes.byref(routed), ctypes.byref(shared) if shared else None)


def moe_route(x: torch.Tensor, w_router: torch.Tensor, k: int, logits: torch.Tensor, topk_idx: torch.Tensor,
              topk_w: torch.Tensor, stream=None) -> None:
    t, h = x.shape
    E = w_router.shape[0]
    _check(lib().moe_route(_ptr(x), _ptr(w_router), t, h, E, k, _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                           _stream(stream)))


def moe_build_csr(topk_idx: torch.Tensor, topk_w: torch.Tensor, E: int, offsets: torch.Tensor,
                  csr_rows: torch.Tensor, csr_w: torch.Tensor, csr_pos: torch.Tensor, workspace: torch.Tensor,
                  stream=None) -> None:
    t, k = topk_idx.shape
    _check(lib().moe_build_csr(_ptr(topk_idx), _ptr(topk_w), t, k, E, _ptr(offsets), _ptr(csr_rows), _ptr(csr_w),
                               _ptr(csr_pos), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)))


def moe_shared(x: torch.Tensor, layout: moe_layout, record: torch.Tensor, gate_w: Optional[torch.Tensor],
               out: torch.Tensor, accumulate: int, workspace: torch.Tensor, stream=None) -> None:
    t = x.shape[0]
    _check(lib().moe_shared(_ptr(x), t, ctypes.byref(layout), _ptr(record), _ptr(gate_w), _ptr(out), accumulate,
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


class MoeRing:
    """Owner of a moe_ring handle (events, copy stream); slots are caller memory."""

    def __init__(self, layout: moe_layout, slots: torch.Tensor, n_slots: int = 64, group: int = 8):
        self._h = ctypes.c_void_p()
        self.slots = slots
        _check(lib().moe_ring_create(ctypes.byref(layout), _ptr(slots), n_slots, group, ctypes.byref(self._h)))

    @property
    def handle(self):
        return self._h

    def set_miss_layout(self, miss_layout: Optional[moe_layout], staging: Optional[torch.Tensor]):
        """Streamed records in the 2-bit layout `miss_layout`, staged in
        `staging` (n_slots * miss stride bytes on the device); None: 4-bit."""
        self.staging = staging
        _check(lib().moe_ring_set_miss_layout(self._h, ctypes.byref(miss_layout) if miss_layout is not None else None,
                                              _ptr(staging)))

    def stats(self) -> dict:
        s = moe_ring_stats()
        _check(lib().moe_ring_get_stats(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in s._fields_}

    def close(self):
        if self._h:
            lib().moe_ring_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_prefill_experts(x: torch.Tensor, k: int, E: int, layout: moe_layout, offsets: torch.Tensor,
                        csr_rows: torch.Tensor, csr_w: torch.Tensor, csr_pos: torch.Tensor, records: torch.Tensor,
                        out: torch.Tensor, accumulate: int, workspace: torch.Tensor,
                        host_records: Optional[Sequence[Optional[torch.Tensor]]] = None,
                        ring: Optional[MoeRing] = None, stream=None) -> None:
    t = x.shape[0]
    hr = None
    if host_records is not None:
        hr = (ctypes.c_void_p * E)(*[(r.data_ptr() if r is not None else None) for r in host_records])
    _check(lib().moe_prefill_experts(_ptr(x), t, k, E, ctypes.byref(layout), _ptr(offsets), _ptr(csr_rows),
                                     _ptr(csr_w), _ptr(csr_pos), _ptr(records), hr,
                                     ring.handle if ring is not None else None, _ptr(out), accumulate,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def moe_prefill_fused(x: torch.Tensor, k: int, E: int, layout: moe_layout, offsets: torch.Tensor,
                      csr_rows: torch.Tensor, csr_w: torch.Tensor, csr_pos: torch.Tensor, records: torch.Tensor,
                      shared_layout: moe_layout, shared_record: torch.Tensor, shared_gate_w: Optional[torch.Tensor],
                      out: torch.Tensor, accumulate: int, workspace: torch.Tensor, stream=None) -> None:
    t = x.shape[0]
    _check(lib().moe_prefill_fused(_ptr(x), t, k, E, ctypes.byref(layout), _ptr(offsets), _ptr(csr_rows),
                                   _ptr(csr_w), _ptr(csr_pos), _ptr(records), ctypes.byref(shared_layout),
                                   _ptr(shared_record), _ptr(shared_gate_w), _ptr(out), accumulate,
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def moe_block(x: torch.Tensor, w_router: torch.Tensor, k: int, layout: moe_layout, records: torch.Tensor,
              shared_layout: Optional[moe_layout], shared_record: Optional[torch.Tensor],
              shared_gate_w: Optional[torch.Tensor], logits: torch.Tensor, topk_idx: torch.Tensor,
              topk_w: torch.Tensor, offsets: torch.Tensor, csr_rows: torch.Tensor, csr_w: torch.Tensor,
              csr_pos: torch.Tensor, out: torch.Tensor, accumulate: int, workspace: torch.Tensor, stream=None) -> None:
    t = x.shape[0]
    E = w_router.shape[0]
    _check(lib().moe_block(_ptr(x), _ptr(w_router), t, k, E, ctypes.byref(layout), _ptr(records),
                           ctypes.byref(shared_layout) if shared_layout is not None else None, _ptr(shared_record),
                           _ptr(shared_gate_w), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(offsets),
                           _ptr(csr_rows), _ptr(csr_w), _ptr(csr_pos), _ptr(out), accumulate, _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_block_noalloc(x: torch.Tensor, w_router: torch.Tensor, k: int, layout: moe_layout, records: torch.Tensor,
                      shared_layout: Optional[moe_layout], shared_record: Optional[torch.Tensor],
                      shared_gate_w: Optional[torch.Tensor], logits: torch.Tensor, topk_idx: torch.Tensor,
                      topk_w: torch.Tensor, offsets: torch.Tensor, csr_rows: torch.Tensor, csr_w: torch.Tensor,
                      csr_pos: torch.Tensor, out: torch.Tensor, accumulate: int, stream=None) -> None:
    """moe_block on the library's static scratch instead of a workspace."""
    t = x.shape[0]
    E = w_router.shape[0]
    _check(lib().moe_block_noalloc(_ptr(x), _ptr(w_router), t, k, E, ctypes.byref(layout), _ptr(records),
                                   ctypes.byref(shared_layout) if shared_layout is not None else None,
                                   _ptr(shared_record), _ptr(shared_gate_w), _ptr(logits), _ptr(topk_idx),
                                   _ptr(topk_w), _ptr(offsets), _ptr(csr_rows), _ptr(csr_w), _ptr(csr_pos),
                                   _ptr(out), accumulate, _stream(stream)))


def next_norm(hyper: torch.Tensor, alpha: Sequence[float], beta: Sequence[float], gamma: torch.Tensor,
              eps: float, mixed: torch.Tensor) -> moe_next_norm:
    """Describe the next fused norm: hyper fp32 [t, n, h] (updated in place),
    per-copy read / injection weights, gain gamma fp32 [h], output mixed
    bf16 [t, h]."""
    n = hyper.shape[1]
    if len(alpha) != n or len(beta) != n or n > MAX_HC:
        raise ValueError("alpha and beta need one value per residual copy (at most 16)")
    d = moe_next_norm()
    d.hyper = _ptr(hyper)
    d.n = n
    for i in range(n):
        d.alpha[i] = float(alpha[i])
        d.beta[i] = float(beta[i])
    d.gamma = _ptr(gamma)
    d.eps = float(eps)
    d.mixed = _ptr(mixed)
    return d


def moe_inject_norm(y: Optional[torch.Tensor], t: int, h: int, nn: moe_next_norm, stream=None) -> None:
    _check(lib().moe_inject_norm(_ptr(y), t, h, ctypes.byref(nn), _stream(stream)))


def moe_block_next_norm(x: torch.Tensor, w_router: torch.Tensor, k: int, layout: moe_layout, records: torch.Tensor,
                        shared_layout: Optional[moe_layout], shared_record: Optional[torch.Tensor],
                        shared_gate_w: Optional[torch.Tensor], logits: torch.Tensor, topk_idx: torch.Tensor,
                        topk_w: torch.Tensor, offsets: torch.Tensor, csr_rows: torch.Tensor, csr_w: torch.Tensor,
                        csr_pos: torch.Tensor, nn: moe_next_norm, workspace: torch.Tensor, stream=None) -> None:
    t = x.shape[0]
    E = w_router.shape[0]
    _check(lib().moe_block_next_norm(_ptr(x), _ptr(w_router), t, k, E, ctypes.byref(layout), _ptr(records),
                                     ctypes.byref(shared_layout) if shared_layout is not None else None,
                                     _ptr(shared_record), _ptr(shared_gate_w), _ptr(logits), _ptr(topk_idx),
                                     _ptr(topk_w), _ptr(offsets), _ptr(csr_rows), _ptr(csr_w), _ptr(csr_pos),
                                     ctypes.byref(nn), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def moe_residency(offsets: torch.Tensor, budget: int, order: torch.Tensor, keep: torch.Tensor, stream=None) -> None:
    """Experts ranked by row count on the GPU: order int32 [E], keep uint8 [E]."""
    E = offsets.numel() - 1
    _check(lib().moe_residency(_ptr(offsets), E, budget, _ptr(order), _ptr(keep), _stream(stream)))


CHUNK_STATS_FIELDS = ["tokens", "assignments", "experts_touched", "rows_max", "rows_min", "rows_median"]


def moe_chunk_stats_fill(offsets: torch.Tensor, t: int, stats: torch.Tensor, stream=None) -> None:
    """Row statistics of a grouped chunk into `stats` (int32 [8] on the
    device, the fields of CHUNK_STATS_FIELDS then two pad words)."""
    if stats.numel() * stats.element_size() < 32:
        raise ValueError("stats needs 32 bytes")
    E = offsets.numel() - 1
    _check(lib().moe_chunk_stats_fill(_ptr(offsets), t, E, _ptr(stats), _stream(stream)))


def chunk_stats(offsets: torch.Tensor, t: int, stream=None) -> dict:
    """moe_chunk_stats_fill, then the fields read back (synchronises)."""
    stats = torch.empty(8, dtype=torch.int32, device=offsets.device)
    moe_chunk_stats_fill(offsets, t, stats, stream)
    v = stats.cpu().numpy().view("uint32")
    return {f: int(v[i]) for i, f in enumerate(CHUNK_STATS_FIELDS)}


def moe_debug_read_probe(src: torch.Tensor, blocks: int, sink: torch.Tensor, stream=None) -> None:
    """One launch reading all of `src` (the HBM read probe); sink int32 [blocks]."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() < blocks:
        raise ValueError("sink needs one word per workgroup")
    st = lib().moe_debug_read_probe(_ptr(src), nbytes, blocks, _ptr(sink), _stream(stream))
    if st != 0:
        raise MoeError(st, "read probe: bad arguments" if st == 1 else "read probe: launch failed")


def moe_debug_xcc_map(blocks: int, device=None, stream=None):
    """The XCC id of each of `blocks` workgroups of one launch (synchronises)."""
    xcc = torch.full((blocks,), -1, dtype=torch.int32, device=device or "cuda")
    st = lib().moe_debug_xcc_map(_ptr(xcc), blocks, _stream(stream))
    if st != 0:
        raise MoeError(st, "xcc map: bad arguments" if st == 1 else "xcc map: launch failed")
    return xcc.cpu().numpy().view("uint32")


def moe_debug_tile_wait(spins: int = 0, extra: int = 0):
    """Poll limit and forced shortfall of the merged launch's tile wait
    (0, 0: normal operation); see moe_debug_tile_wait in moe_debug.h."""
    st = lib().moe_debug_tile_wait(spins, extra)
    if st != 0:
        raise MoeError(st, "tile wait: bad arguments")


def moe_debug_schedule(offsets: torch.Tensor, bm: int, rows_bound: int, records: torch.Tensor,
                       shared_rec: Optional[int], shared_p0: int, shared_n: int, sched_n: torch.Tensor,
                       order: torch.Tensor, xcap: int, stream=None) -> None:
    """The tile schedule alone (see include/moe_debug.h): sched_n int32 [16],
    order int32 [8 * xcap * 8] (32-byte entries)."""
    E = offsets.numel() - 1
    if sched_n.numel() * sched_n.element_size() < 64 or order.numel() * order.element_size() < 8 * xcap * 32:
        raise ValueError("sched_n needs 64 bytes and order 8 * xcap * 32 bytes")
    st = lib().moe_debug_schedule(_ptr(offsets), E, bm, rows_bound, _ptr(records), shared_rec, shared_p0, shared_n,
                                  _ptr(sched_n), _ptr(order), xcap, _stream(stream))
    if st != 0:
        raise MoeError(st, "schedule: bad arguments" if st == 1 else "schedule: launch failed")


def moe_lookahead(x: torch.Tensor, w_router_next: torch.Tensor, k: int, budget: int, logits: torch.Tensor,
                  topk_idx: torch.Tensor, topk_w: torch.Tensor, counts: torch.Tensor, order: torch.Tensor,
                  keep: torch.Tensor, stream=None) -> None:
    """The next layer's routing on this block's input and its residency by use."""
    t, h = x.shape
    E = w_router_next.shape[0]
    _check(lib().moe_lookahead(_ptr(x), _ptr(w_router_next), t, h, E, k, budget, _ptr(logits), _ptr(topk_idx),
                               _ptr(topk_w), _ptr(counts), _ptr(order), _ptr(keep), _stream(stream)))


def moe_block_from_residual(pending_y: Optional[torch.Tensor], in_norm: moe_next_norm, w_router: torch.Tensor,
                            t: int, k: int, layout: moe_layout, records: torch.Tensor,
                            shared_layout: Optional[moe_layout], shared_record: Optional[torch.Tensor],
                            shared_gate_w: Optional[torch.Tensor], logits: torch.Tensor, topk_idx: torch.Tensor,
                            topk_w: torch.Tensor, offsets: torch.Tensor, csr_rows: torch.Tensor, csr_w: torch.Tensor,
                            csr_pos: torch.Tensor, out_norm: Optional[moe_next_norm], out: Optional[torch.Tensor],
                            accumulate: int, workspace: torch.Tensor, stream=None) -> None:
    """The MoE sub-layer from the residual copies: input norm, block, output (or next norm)."""
    E = w_router.shape[0]
    _check(lib().moe_block_from_residual(_ptr(pending_y), ctypes.byref(in_norm), _ptr(w_router), t, k, E,
                                         ctypes.byref(layout), _ptr(records),
                                         ctypes.byref(shared_layout) if shared_layout is not None else None,
                                         _ptr(shared_record), _ptr(shared_gate_w), _ptr(logits), _ptr(topk_idx),
                                         _ptr(topk_w), _ptr(offsets), _ptr(csr_rows), _ptr(csr_w), _ptr(csr_pos),
                                         ctypes.byref(out_norm) if out_norm is not None else None, _ptr(out),
                                         accumulate, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream)))


def moe_ring_plan_debug(offsets, resident, n_slots: int = 64, group: int = 8):
    """Host-only ring schedule (numpy in, numpy out): slot[E], batch[E], wait[batches]."""
    import numpy as np

    offsets = np.ascontiguousarray(offsets, dtype=np.uint32)
    resident = np.ascontiguousarray(resident, dtype=np.uint64)
    E = offsets.size - 1
    slot = np.empty(E, np.int32)
    batch = np.empty(E, np.int32)
    wait = np.empty(max(E, 1), np.int32)
    nb = lib().moe_ring_plan_debug(offsets.ctypes.data, resident.ctypes.data, E, n_slots, group,
                                   slot.ctypes.data, batch.ctypes.data, wait.ctypes.data)
    return slot, batch, wait[:nb]


def moe_profile_begin(phases: Sequence[str]) -> None:
    """Start timing every kernel of the named phases (see PHASES) with HIP events."""
    mask = 0
    for p in phases:
        mask |= 1 << PHASES.index(p)
    lib().moe_profile_begin(mask)


def moe_profile_set_mask(phases: Sequence[str]) -> None:
    """Time the named phases from now on, keeping what was recorded so far ([] pauses)."""
    mask = 0
    for p in phases:
        mask |= 1 << PHASES.index(p)
    lib().moe_profile_set_mask(mask)


def moe_profile_end() -> dict:
    """Stop timing; returns {phase: (total_ms, launches)} for phases that ran."""
    import numpy as np

    ms = np.zeros(len(PHASES), np.float64)
    n = np.zeros(len(PHASES), np.int64)
    if lib().moe_profile_end(ms.ctypes.data, n.ctypes.data) < 0:
        raise MoeError(4, "profile events failed")
    return {p: (float(ms[i]), int(n[i])) for i, p in enumerate(PHASES) if n[i]}


from .block import MoeBlock  # noqa: E402  (device-buffer owner built on the calls above)
