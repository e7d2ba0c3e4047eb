"""Device buffers for one MoE block and its calls in their order.

Owns the GPU tensors of one layer shape (inputs, routing outputs, CSR,
workspace, output) and runs

    moe_shared(accumulate=0) -> moe_route -> moe_build_csr -> moe_prefill_experts(accumulate=1)

the order of the cherenkov experts.rs page (fn pf_experts: shared expert into
the zeroed output, then routed experts added in ascending id), or, when the
shared record has the routed layout and every expert is resident,

    moe_route -> moe_build_csr -> moe_prefill_fused(accumulate=0)

which runs the shared expert inside the routed experts' grouped launches and
adds its term first in the combine.  In the separate form the shared expert
needs no routing, so forward() can run it on a second stream of the same
(default) priority while routing and grouping run; the routed call waits for
it, so every row still receives the shared term first.  Only allocation and
call sequencing live here; the arithmetic is in libmoe.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import (MoeRing, chunk_stats, moe_block, moe_block_next_norm, moe_block_noalloc, moe_build_csr,
               moe_layout_make, moe_layout_make_bits, moe_prefill_experts, moe_prefill_fused, moe_route, moe_shared,
               moe_workspace_bytes)


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on device (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


class MoeBlock:
    def __init__(self, t: int, hidden: int, inter: int, inter_shared: Optional[int], experts: int, k: int,
                 group: int, device="cuda"):
        self.t, self.h, self.I, self.E, self.k, self.G = t, hidden, inter, experts, k, group
        self.Is = inter_shared
        self.device = torch.device(device)
        self.L = moe_layout_make(hidden, inter, group)
        self.Ls = moe_layout_make(hidden, inter_shared, group) if inter_shared else None
        d = self.device
        self.logits = torch.empty((t, experts), dtype=torch.float32, device=d)
        self.topk_idx = torch.empty((t, k), dtype=torch.int32, device=d)
        self.topk_w = torch.empty((t, k), dtype=torch.float32, device=d)
        self.offsets = torch.empty(experts + 1, dtype=torch.int32, device=d)
        self.csr_rows = torch.empty(t * k, dtype=torch.int32, device=d)
        self.csr_w = torch.empty(t * k, dtype=torch.float32, device=d)
        self.csr_pos = torch.empty(t * k, dtype=torch.int32, device=d)
        self.out = torch.empty((t, hidden), dtype=torch.float32, device=d)
        nbytes = moe_workspace_bytes(t, k, experts, self.L, self.Ls)
        if nbytes == 0:
            raise ValueError("invalid block shape")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=d)
        self.x = self.w_router = self.pool = self.table = self.shared_record = self.gate_w = None
        self.host_records: Optional[Sequence[Optional[torch.Tensor]]] = None
        self.ring: Optional[MoeRing] = None
        self._side = torch.cuda.Stream(device=d) if d.type == "cuda" else None
        self._fork = torch.cuda.Event() if d.type == "cuda" else None
        self._join = torch.cuda.Event() if d.type == "cuda" else None

    @classmethod
    def from_workload(cls, wl, device="cuda", resident: Optional[np.ndarray] = None, ring_slots: int = 64,
                      group: int = 8, shared: bool = True, miss_records: Optional[np.ndarray] = None):
        """Upload a moe_synth workload.  resident[e] False -> expert e streams
        through a ring (as its 2-bit record miss_records[e] when given)."""
        c = wl.cfg
        b = cls(wl.x.shape[0], c.hidden, c.inter, c.inter_shared if shared else None, c.experts, c.k, c.group, device)
        b.set_inputs(wl.x, wl.w_router)
        b.set_records(wl.records, resident, ring_slots, group, miss_records)
        if shared:
            b.set_shared(wl.shared_record, wl.gate_w)
        return b

    def set_inputs(self, x_bits: np.ndarray, w_router: np.ndarray):
        self.x = bf16_tensor(x_bits, self.device)
        self.w_router = torch.from_numpy(np.ascontiguousarray(w_router, dtype=np.float32)).to(self.device)

    def set_records(self, records: np.ndarray, resident: Optional[np.ndarray] = None, ring_slots: int = 64,
                    group: int = 8, miss_records: Optional[np.ndarray] = None):
        """records [E, stride]: 4-bit records; resident[e] False streams expert e
        through a ring, from miss_records[e] (2-bit, [E, miss stride]) when
        given, else from records[e]."""
        E, stride = records.shape
        assert stride == self.L.stride and E == self.E
        if resident is None:
            resident = np.ones(E, dtype=bool)
        res_ids = np.nonzero(resident)[0]
        self.pool = torch.from_numpy(np.ascontiguousarray(records[res_ids])).to(self.device)
        table = np.zeros(E, dtype=np.int64)
        base = self.pool.data_ptr()
        table[res_ids] = base + np.arange(res_ids.size, dtype=np.int64) * stride
        self.table = torch.from_numpy(table).to(self.device)
        if resident.all():
            self.host_records, self.ring = None, None
            return
        src = records if miss_records is None else miss_records
        # the streamed records in one pinned buffer, in expert order, so the
        # ring can copy runs of consecutive experts at once
        ids = np.nonzero(~resident)[0]
        self.host_pool = torch.empty((ids.size, src.shape[1]), dtype=torch.uint8).pin_memory()
        self.host_pool.numpy()[:] = src[ids]
        self.host_records = [None] * E
        for i, e in enumerate(ids):
            self.host_records[e] = self.host_pool[i]
        self.ring_slots = torch.empty((ring_slots, stride), dtype=torch.uint8, device=self.device)
        self.ring = MoeRing(self.L, self.ring_slots, ring_slots, group)
        if miss_records is not None:
            self.Lmiss = moe_layout_make_bits(self.h, self.I, self.G, 2)
            assert miss_records.shape[1] == self.Lmiss.stride
            staging = torch.empty((ring_slots, self.Lmiss.stride), dtype=torch.uint8, device=self.device)
            self.ring.set_miss_layout(self.Lmiss, staging)

    def set_pool(self, pool: torch.Tensor):
        """Every expert resident in `pool`, a device uint8 tensor [E, stride]
        holding record e at row e (records of experts that no row picks are
        never read)."""
        same_device = pool.device.type == self.device.type and (
            self.device.index is None or pool.device.index == self.device.index)
        if not same_device or pool.dtype != torch.uint8 or tuple(pool.shape) != (self.E, self.L.stride):
            raise ValueError("pool must be a uint8 [E, stride] tensor on the block's device")
        self.pool = pool
        self.table = pool.data_ptr() + torch.arange(self.E, dtype=torch.int64, device=self.device) * self.L.stride
        self.host_records, self.ring = None, None

    def use_ring(self, ring_slots: int = 64, group: int = 8):
        """Run the all-resident records through a ring too (every batch gated by events)."""
        self.ring_slots = torch.empty((ring_slots, self.L.stride), dtype=torch.uint8, device=self.device)
        self.ring = MoeRing(self.L, self.ring_slots, ring_slots, group)
        self.host_records = [None] * self.E

    def set_shared(self, record: np.ndarray, gate_bits: Optional[np.ndarray] = None):
        self.shared_record = torch.from_numpy(np.ascontiguousarray(record)).to(self.device)
        self.gate_w = None if gate_bits is None else bf16_tensor(gate_bits, self.device)

    # ---------------------------------------------------------------- calls
    def route(self, stream=None):
        moe_route(self.x, self.w_router, self.k, self.logits, self.topk_idx, self.topk_w, stream)

    def build_csr(self, stream=None):
        moe_build_csr(self.topk_idx, self.topk_w, self.E, self.offsets, self.csr_rows, self.csr_w, self.csr_pos,
                      self.workspace, stream)

    def chunk_stats(self, stream=None) -> dict:
        """Report of the last call (prefill.rs page, struct ChunkStats): its
        rows and the grouping's expert-row statistics (moe_chunk_stats_fill),
        and the records fetched over the host link, their bytes and the
        host's wait for ring slots, all 0 when every expert is resident.
        Synchronises."""
        st = chunk_stats(self.offsets, self.t, stream)
        rs = self.ring.stats() if self.ring is not None else None
        st["fetched"] = rs["streamed"] if rs else 0
        st["fetched_bytes"] = rs["fetched_bytes"] if rs else 0
        st["wait_s"] = rs["wait_ms"] / 1e3 if rs else 0.0
        return st

    def shared(self, accumulate: int = 0, stream=None):
        moe_shared(self.x, self.Ls, self.shared_record, self.gate_w, self.out, accumulate, self.workspace, stream)

    def fused(self, accumulate: int = 0, stream=None):
        moe_prefill_fused(self.x, self.k, self.E, self.L, self.offsets, self.csr_rows, self.csr_w, self.csr_pos,
                          self.table, self.Ls, self.shared_record, self.gate_w, self.out, accumulate, self.workspace,
                          stream)

    def block(self, accumulate: int = 0, stream=None):
        moe_block(self.x, self.w_router, self.k, self.L, self.table, self.Ls, self.shared_record, self.gate_w,
                  self.logits, self.topk_idx, self.topk_w, self.offsets, self.csr_rows, self.csr_w, self.csr_pos,
                  self.out, accumulate, self.workspace, stream)

    def block_next_norm(self, nn, stream=None):
        """The one-call block with its output injected into the next fused
        norm (`nn` from mixture_experts_prefill_amd.next_norm) instead of
        written to out."""
        moe_block_next_norm(self.x, self.w_router, self.k, self.L, self.table, self.Ls, self.shared_record,
                            self.gate_w, self.logits, self.topk_idx, self.topk_w, self.offsets, self.csr_rows,
                            self.csr_w, self.csr_pos, nn, self.workspace, stream)

    def block_noalloc(self, accumulate: int = 0, stream=None):
        """The one-call block on the library's static scratch (no workspace)."""
        moe_block_noalloc(self.x, self.w_router, self.k, self.L, self.table, self.Ls, self.shared_record,
                          self.gate_w, self.logits, self.topk_idx, self.topk_w, self.offsets, self.csr_rows,
                          self.csr_w, self.csr_pos, self.out, accumulate, stream)

    @property
    def can_block(self) -> bool:
        """Every expert resident, and no shared expert or one of the routed layout."""
        return self.ring is None and self.host_records is None and (self.Ls is None or self.can_fuse)

    @property
    def can_fuse(self) -> bool:
        """The shared record has the routed layout and no expert streams through a ring."""
        return (self.Ls is not None and self.ring is None and self.host_records is None
                and (self.Ls.hidden, self.Ls.inter, self.Ls.group) == (self.L.hidden, self.L.inter, self.L.group))

    def experts(self, accumulate: int = 1, stream=None):
        moe_prefill_experts(self.x, self.k, self.E, self.L, self.offsets, self.csr_rows, self.csr_w, self.csr_pos,
                            self.table, self.out, accumulate, self.workspace, self.host_records, self.ring, stream)

    # Rows from which the shared expert runs on a second stream beside the
    # routing calls.  The fork and join cost about 10 us each of cross-queue
    # latency on MI355X, while below this the two chains are short
    # latency-bound kernels (measured: t = 1 and 8 run faster in one stream,
    # t = 512 and 4096 faster forked).
    FORK_MIN_ROWS = 64

    def forward(self, stream=None, fork: Optional[bool] = None, fused: Optional[bool] = None,
                path: Optional[str] = None) -> torch.Tensor:
        """One block.  `stream` (torch stream, raw handle or None for the current
        stream) carries routing, grouping and the routed experts.  `path`:
          "block"    the whole block in one call (moe_block), the default
                     whenever can_block;
          "fused"    moe_route, moe_build_csr, moe_prefill_fused (fused=True);
          "separate" the shared expert in its own call (fused=False, and the
                     default with a ring): with `fork` (default:
                     t >= FORK_MIN_ROWS) it forks off the stream onto a second
                     one and joins back before the routed call, otherwise it
                     runs first on the same stream."""
        if path is None:
            if fused is None:
                path = "block" if self.can_block else "separate"
            else:
                path = "fused" if fused else "separate"
        if fork is None:
            fork = self.t >= self.FORK_MIN_ROWS
        if path == "block":
            if not self.can_block:
                raise ValueError("one-call block needs resident experts and a shared record of the routed layout")
            self.block(0, stream)
            return self.out
        fused = path == "fused"
        if fused:
            if not self.can_fuse:
                raise ValueError("fused block needs a shared record of the routed layout and resident experts")
            self.route(stream)
            self.build_csr(stream)
            self.fused(0, stream)
        elif self.Ls is not None and not fork:
            self.shared(0, stream)
            self.route(stream)
            self.build_csr(stream)
            self.experts(1, stream)
        elif self.Ls is not None:
            if stream is None:
                main = torch.cuda.current_stream(self.device)
            elif isinstance(stream, torch.cuda.Stream):
                main = stream
            else:
                main = torch.cuda.ExternalStream(int(stream), device=self.device)
            self._fork.record(main)
            self._side.wait_event(self._fork)
            self.shared(0, self._side)
            self._join.record(self._side)
            self.route(main)
            self.build_csr(main)
            main.wait_event(self._join)
            self.experts(1, main)
        else:
            self.route(stream)
            self.build_csr(stream)
            self.experts(0, stream)
        return self.out
