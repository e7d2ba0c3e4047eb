"""Benchmark of the routed-expert MoE prefill block on one MI355X.

One step = one whole block over one chunk, on inputs already resident in
HBM: moe_block (routing, grouping, routed and shared experts in one call), or
with --separate moe_shared -> moe_route -> moe_build_csr -> moe_prefill_experts.
Default workload: the full prefill chunk (t = 4096 rows, hidden 2048, expert
inter 768, 128 experts, top-8, shared expert inter 768, 4-bit group-64
weights, Zipf(1.1) expert popularity).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config full|mid|decode|decode1|large|tiny]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MALL_BYTES = 256 << 20      # MI355X Infinity Cache (last-level cache in front of HBM)
METRIC = "MoE-layer prefill tokens/sec at t=4096; % of bf16 MFMA / HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The dominant kernel's sources: the GEMM file, the headers whose code it
# compiles, the function that orders its tiles (schedule_body in csr.hip: the
# order decides which weights and rows are still in L2, so the traffic), and
# the parts of the shared internal header it reads (its argument and
# tile-entry structs and the tiling constants); the API declarations and the
# other kernels around them do not change the GEMM.
KERNEL_SOURCES = ["mixture_experts_prefill_amd/csrc/gemm.hip", "mixture_experts_prefill_amd/csrc/lds_dma.h",
                  "mixture_experts_prefill_amd/csrc/profile.h"]
SCHEDULE_SOURCE = "mixture_experts_prefill_amd/csrc/csr.hip"
KERNEL_HEADER = "mixture_experts_prefill_amd/csrc/moe_internal.h"


def source_hash() -> str:
    """Hash of the dominant kernel's sources with comments and blank space
    removed, so that its counters stay attached to the code they were taken
    on, not to its prose or to the other kernels."""
    import re

    def strip(text):
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        return " ".join(text.split())

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(f.encode() + strip(fh.read()).encode())
    with open(os.path.join(ROOT, SCHEDULE_SOURCE), encoding="utf-8") as fh:
        sch = strip(fh.read())
    m = re.search(r"template <int MAXT> __device__ __forceinline__ void schedule_body\(.*?sched_n\[0\] = T; \}", sch)
    h.update(SCHEDULE_SOURCE.encode() + (m.group(0) if m else sch).encode())
    with open(os.path.join(ROOT, KERNEL_HEADER), encoding="utf-8") as fh:
        hdr = strip(fh.read())
    parts = re.findall(r"struct (?:GemmArgs|TileEntry) \{.*?\};", hdr) + re.findall(r"constexpr int k\w+ = [^;]*;", hdr)
    h.update(KERNEL_HEADER.encode() + " ".join(parts).encode())
    return h.hexdigest()[:16]


def algorithmic(cfg, t, counts, fused=False):
    """FLOPs and bytes the method itself must do (no padding, no intermediates).
    With `fused` the shared expert's gate/up and down run inside the routed
    launches, so their work is counted there (and flop_shared is 0)."""
    import numpy as np

    h, I, Is, E, k = cfg.hidden, cfg.inter, cfg.inter_shared, cfg.experts, cfg.k
    import moe_synth as ms

    R = ms.layout(h, I, cfg.group).stride
    Rs = ms.layout(h, Is, cfg.group).stride
    touched = int((np.asarray(counts) > 0).sum())
    gu_weights = 2 * (h * I // 2 + h * I // cfg.group * 4)   # gate + up codes and scale/bias of one record
    gu_weights_s = 2 * (h * Is // 2 + h * Is // cfg.group * 4)
    dn_weights = h * I // 2 + h * I // cfg.group * 4         # down codes and scale/bias of one record
    dn_weights_s = h * Is // 2 + h * Is // cfg.group * 4
    sh = 1.0 if fused else 0.0
    return dict(
        flop_gateup=4.0 * t * k * h * I + sh * 4.0 * t * h * Is,
        # gate/up kernel: weights of the touched experts (and the shared
        # expert's when fused), x rows once, SiLU*up written once
        bytes_gateup=touched * gu_weights + sh * gu_weights_s + 2.0 * t * h + 2.0 * t * k * I + sh * 2.0 * t * Is,
        flop_down=2.0 * t * k * h * I + sh * 2.0 * t * h * Is,
        # down kernel: down weights of the touched experts (and the shared
        # expert's when fused), SiLU*up read once, ye written once
        bytes_down=touched * dn_weights + sh * dn_weights_s + 2.0 * t * k * I + sh * 2.0 * t * Is
                   + 2.0 * t * k * h + sh * 2.0 * t * h,
        flop_shared=(1.0 - sh) * 6.0 * t * h * Is,
        flop_router=2.0 * t * h * E,
        bytes_total=touched * R + Rs + 4.0 * E * h + 2.0 * t * h + 4.0 * t * h,
        touched=touched,
    )


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# The dominant kernel: the merged grouped gate/up + down launch where the
# block uses it (moe_block and moe_prefill_fused, chunks of more than two
# rows), else the grouped gate/up kernel (any tile height; 4 waves).
MERGED_KERNEL = "k_gemm_gu_down"
GATEUP_KERNEL = "k_gemm<0,"
COPY_PROBE_BYTES = 512 << 20
READ_PROBE_BYTES = 2 << 30     # read once by the HBM read probe: 8x the MALL
READ_PROBE_BLOCKS = 16384


def traffic_for(kernel_key: str):
    """HBM bytes per launch from the committed counter runs, if they match this build."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def ingest_pmc(fetch_csv: str, write_csv: str, config: str, separate: bool):
    """Per-launch HBM bytes of the dominant kernel from two rocprofv3 --pmc runs.

    Each counter (KiB per dispatch) is scaled by the ratio of known bytes to
    what the same counter reads for the copy probe (a device-to-device copy of
    COPY_PROBE_BYTES, which reads and writes that many bytes once).  The
    dominant kernel is the merged gate/up + down launch when the run has it,
    else the gate/up launch.
    """
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    merged = any(MERGED_KERNEL in k for k in per_kernel(fetch_csv, "FETCH_SIZE"))
    kernel = MERGED_KERNEL if merged else GATEUP_KERNEL
    key = ("experts_" if merged else "gateup_") + config + ("_separate" if separate else "")
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        dom = [v for k, vs in vals.items() if kernel in k for v in vs]
        cp = [v for k, vs in vals.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs
              if v * 1024 > COPY_PROBE_BYTES / 2]
        if not dom or not cp:
            raise SystemExit(f"{counter}: dominant kernel or copy probe missing from {path}")
        factor = COPY_PROBE_BYTES / (max(cp) * 1024)
        out[counter] = dict(kib_per_launch=sum(dom) / len(dom), copy_kib=max(cp), factor=factor,
                            bytes_per_launch=sum(dom) / len(dom) * 1024 * factor)
    entry = dict(kernel=kernel, source_hash=source_hash(),
                 fetch_bytes=round(out["FETCH_SIZE"]["bytes_per_launch"]),
                 write_bytes=round(out["WRITE_SIZE"]["bytes_per_launch"]),
                 bytes_per_launch=round(out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]),
                 fetch_factor=round(out["FETCH_SIZE"]["factor"], 4), write_factor=round(out["WRITE_SIZE"]["factor"], 4),
                 raw=out)
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data[key] = entry
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=2)
    print(json.dumps({key: {k: v for k, v in entry.items() if k != "raw"}}, indent=2))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg_name: str, rows: int, rows_1t: int):
    """The oracle, as it stands, on the first `rows` rows of the same workload
    with all its threads, and on the first `rows_1t` rows with one thread."""
    import dataclasses

    import moe_synth as ms
    import oracle

    full = ms.make_workload(cfg_name)

    def sample(n):
        return dataclasses.replace(full, x=full.x[:n].copy(), cfg=dataclasses.replace(full.cfg, t=n))

    wl = sample(rows)
    threads = oracle.max_threads()
    # repeated until about 10 s of CPU work (at most 3 runs), for a stable rate
    times = []
    while len(times) < 3 and sum(times) < 10.0:
        t0 = time.perf_counter()
        oracle.block(wl, with_logits=False)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    one = None
    if rows_1t > 0:
        oracle.set_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.block(sample(rows_1t), with_logits=False)
            dt1 = time.perf_counter() - t0
        finally:
            oracle.set_threads(threads)
        one = {"value": round(rows_1t / dt1, 2), "unit": "tokens/s", "cores": 1,
               "sample": f"first {rows_1t} rows, one run of {dt1:.2f} s (the touched experts' weights are "
                         f"decoded once per call, so a small sample has a lower rate per row)"}
    return {"value": round(rows / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"full block (router, top-k, CSR, routed experts, shared expert, combine) in double "
                      f"on the first {rows} of {cfg_name}'s {ms.CONFIGS[cfg_name].t} rows, {len(times)} runs "
                      f"of {dt:.2f} s on average",
            "single_thread": one}


def build_block(cfg, all_resident: bool, miss_bits: int = 4):
    """Device buffers of one workload.  Every expert resident: routing runs
    once on the GPU and only the records of experts some row picks are
    generated (the others are never read); with cfg.resident and not
    `all_resident`, the most-used experts are resident and the rest stream
    from pinned host memory through the ring."""
    import numpy as np
    import torch

    import mixture_experts_prefill_amd as mep
    import moe_synth as ms

    x = ms.make_x(cfg)
    blk = mep.MoeBlock(cfg.t, cfg.hidden, cfg.inter, cfg.inter_shared, cfg.experts, cfg.k, cfg.group)
    blk.set_inputs(x, ms.make_router(cfg))
    blk.set_shared(ms.make_shared(cfg))
    blk.route()
    blk.build_csr()
    torch.cuda.synchronize()
    counts = np.diff(blk.offsets.cpu().numpy().astype(np.int64))
    touched = np.nonzero(counts > 0)[0]
    resident = None
    if cfg.resident and not all_resident:
        # the most-used experts stay resident: ranked on the GPU from the offsets
        order = torch.empty(cfg.experts, dtype=torch.int32, device="cuda")
        keep = torch.empty(cfg.experts, dtype=torch.uint8, device="cuda")
        mep.moe_residency(blk.offsets, cfg.resident, order, keep)
        resident = keep.cpu().numpy().astype(bool)
        wl = ms.make_workload(cfg)
        miss = None
        if miss_bits == 2:
            # streamed experts cross the host link as 2-bit records
            ids = np.nonzero(~resident)[0]
            miss = np.zeros((cfg.experts, ms.layout(cfg.hidden, cfg.inter, cfg.group, 2).stride), np.uint8)
            miss[ids] = ms.make_records(cfg, experts=ids.tolist(), bits=2)
        blk = mep.MoeBlock.from_workload(wl, resident=resident, miss_records=miss)
        del wl, miss
    else:
        pool = torch.empty((cfg.experts, blk.L.stride), dtype=torch.uint8, device="cuda")
        for i in range(0, touched.size, 32):
            ids = touched[i:i + 32]
            recs = torch.from_numpy(ms.make_records(cfg, experts=ids.tolist()))
            pool[torch.from_numpy(ids).to("cuda")] = recs.to("cuda")
        blk.set_pool(pool)
    return blk, counts, resident


def measure(cfg, args, steps: int, warmup_steps, all_resident: bool = False, separate: bool = False):
    """Time `steps` whole blocks of workload `cfg`; returns the measurements."""
    import numpy as np
    import torch

    import mixture_experts_prefill_amd as mep

    log(f"[bench] workload {cfg.name}: generating and uploading ...")
    blk, counts, resident = build_block(cfg, all_resident, args.miss_bits)
    t = cfg.t
    # Weight copies rotated per step: the experts' records, the router weights
    # and the shared expert's record (a model's layers each have their own).
    copies = args.copies
    if copies <= 0:
        # Between two steps on the same copy, the other copies stream
        # (copies - 1) x the step's weight bytes; make that exceed the MALL.
        touched_bytes = algorithmic(cfg, t, counts)["bytes_total"]
        copies = min(8, max(2, int(MALL_BYTES // touched_bytes) + 2))
    sets = [(blk.table, blk.w_router, blk.shared_record)]
    pools = [blk.pool]
    for c in range(1, copies if resident is None else 1):
        pool = blk.pool.clone()
        pools.append(pool)
        tab = blk.table.clone()
        nz = tab != 0
        tab[nz] = tab[nz] - blk.pool.data_ptr() + pool.data_ptr()
        sets.append((tab, blk.w_router.clone(), blk.shared_record.clone()))

    # the whole block in one call (moe_block) unless the shared expert must run
    # in its own call (--separate, or experts streamed through the ring)
    path = "block" if blk.can_block and not separate else "separate"
    fused = path == "block" and blk.Ls is not None

    def step(i):
        blk.table, blk.w_router, blk.shared_record = sets[i % len(sets)]
        blk.forward(path=path)

    # Untimed warm-up: by default at least 20 steps and 30 ms of GPU work.
    # After only 5 steps the timed ones still ran 5% slower (full chunk 0.513
    # vs 0.483-0.487 ms per step for 20, 50 or 200 warm-up steps).
    warmup = 0
    w_start = time.perf_counter()
    while True:
        n = warmup_steps if warmup_steps is not None else 20
        for _ in range(n if warmup == 0 else 10):
            step(warmup)
            warmup += 1
        torch.cuda.synchronize()
        if warmup_steps is not None or time.perf_counter() - w_start >= 0.03:
            break

    # The dominant kernel's launches are timed with HIP events attached to
    # them (hipExtLaunchKernel) in every `--time-every`-th timed step: the
    # attached events leave ~5 us of idle time on each side of the kernel, so
    # timing every launch would charge that to the step time.
    mep.moe_profile_begin([])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        mep.moe_profile_set_mask(["gateup", "experts"] if i % args.time_every == 0 else [])
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    prof = mep.moe_profile_end()
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / steps
    value = t * steps / (gpu_ms / 1e3)
    log(f"[bench] {cfg.name}: {steps} steps after {warmup} warm-up: {ms_per_step:.4f} ms/step "
        f"(wall {wall * 1e3 / steps:.3f} ms/step)")

    work = algorithmic(cfg, t, counts, fused)
    # The merged gate/up + down launch ("experts") when the block ran it,
    # else the gate/up launch.
    dominant = "experts" if "experts" in prof else "gateup"
    if dominant == "experts":
        dom_flop = work["flop_gateup"] + work["flop_down"]
        dom_bytes = work["bytes_gateup"] + work["bytes_down"]
    else:
        dom_flop, dom_bytes = work["flop_gateup"], work["bytes_gateup"]
    dom_ms, dom_n = prof[dominant]
    dom_avg_s = dom_ms / dom_n / 1e3
    # Launches per step: one, except with streamed experts, where the ring
    # runs the GEMMs once per batch; each launch then does its share.
    timed_steps = len(range(0, steps, args.time_every))
    per_launch = timed_steps / dom_n
    # The kernel is MFMA-bound when its arithmetic intensity exceeds the
    # machine balance (2500 TFLOP/s / 8 TB/s = 312 FLOP/B), else HBM-bound.
    intensity = dom_flop / dom_bytes
    if dominant == "experts":
        kname = ("k_gemm_gu_down: grouped gate/up (SiLU*up epilogue) and down of the routed experts"
                 + (" and the shared expert" if fused else "") + " in one launch, int4 -> bf16 MFMA")
        tkey = f"experts_{cfg.name}" + ("" if fused else "_separate")
    else:
        kname = ("k_gemm gate/up (routed experts and the shared expert in one grouped launch, int4 -> bf16 MFMA, "
                 "SiLU*up epilogue)" if fused else
                 "k_gemm gate/up (routed, grouped int4 -> bf16 MFMA, SiLU*up epilogue)")
        tkey = f"gateup_{cfg.name}" + ("" if fused else "_separate")
    if intensity >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = dom_flop * per_launch / dom_avg_s / 1e12
        roofline = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_for(tkey), "algorithmic": round(dom_flop * per_launch),
                    "avg_launch_us": round(dom_avg_s * 1e6, 2), "launches_per_step": round(1 / per_launch, 2)}
    else:
        achieved = dom_bytes * per_launch / dom_avg_s / 1e9
        roofline = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": traffic_for(tkey), "algorithmic": round(dom_bytes * per_launch),
                    "avg_launch_us": round(dom_avg_s * 1e6, 2), "launches_per_step": round(1 / per_launch, 2)}

    block_flop = work["flop_gateup"] + work["flop_down"] + work["flop_shared"]
    step_s = ms_per_step / 1e3
    extra = {"block_mfma_frac": round(block_flop / step_s / 1e12 / PEAK_BF16_TFLOPS, 4),
             "block_hbm_frac": round(work["bytes_total"] / step_s / 1e9 / PEAK_HBM_GBS, 4),
             "block_algorithmic_flop": round(block_flop), "block_algorithmic_bytes": round(work["bytes_total"]),
             "touched_experts": work["touched"], "max_rows_per_expert": int(counts.max()),
             "weight_copies": len(sets),
             "calls": "moe_block (shared expert in the routed launches)" if path == "block"
                      else "moe_shared, moe_route, moe_build_csr, moe_prefill_experts"}
    if blk.ring is not None:
        # streamed experts: the host link is the bound; the ring counters are
        # those of the last call (one step)
        rs = blk.ring.stats()
        extra["ring"] = {"streamed_experts": rs["streamed"], "batches": rs["batches"], "miss_bits": args.miss_bits,
                         "fetched_bytes_per_step": rs["fetched_bytes"],
                         "h2d_GBps": round(rs["fetched_bytes"] / step_s / 1e9, 2),
                         "host_wait_ms": round(rs["wait_ms"], 3)}
        # the link itself: pinned host -> device copies of 512 MiB
        hsrc = torch.empty(1 << 29, dtype=torch.uint8).pin_memory()
        ddst = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
        ddst.copy_(hsrc, non_blocking=True)
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(3):
            ddst.copy_(hsrc, non_blocking=True)
        c1.record()
        torch.cuda.synchronize()
        probe = 3 * (1 << 29) / (c0.elapsed_time(c1) / 1e3) / 1e9
        extra["ring"]["h2d_probe_GBps"] = round(probe, 2)
        extra["ring"]["h2d_frac_of_probe"] = round(extra["ring"]["h2d_GBps"] / probe, 4)
        del hsrc, ddst

    # Per-step distribution in an extra untimed pass: an event between steps
    # (its own cost is small next to a step, but it is kept out of `value`).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    extra["step_ms_p10_p50_p90"] = [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)]

    if args.next_norm_copies > 0 and path == "block":
        # The block output into the next fused norm (n residual copies): the
        # one-call block then moe_inject_norm on its output, against
        # moe_block_next_norm, which never writes the output.
        nc, hdim = args.next_norm_copies, cfg.hidden
        hyper = torch.randn((t, nc, hdim), device="cuda")
        gamma = torch.ones(hdim, device="cuda")
        mixed = torch.empty((t, hdim), dtype=torch.int16, device="cuda")
        nn = mep.next_norm(hyper, [1.0 / nc] * nc, [1.0] * nc, gamma, 1e-6, mixed)

        def two_calls(i):
            step(i)
            mep.moe_inject_norm(blk.out, t, hdim, nn)

        def fused_call(i):
            blk.table, blk.w_router, blk.shared_record = sets[i % len(sets)]
            blk.block_next_norm(nn)

        nn_ms = {}
        for name, fn in (("block_then_inject_norm", two_calls), ("block_next_norm", fused_call)):
            for i in range(20):
                fn(i)
            n0 = torch.cuda.Event(enable_timing=True)
            n1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            n0.record()
            for i in range(steps):
                fn(i)
            n1.record()
            torch.cuda.synchronize()
            nn_ms[name] = round(n0.elapsed_time(n1) / steps, 4)
        extra["next_norm"] = {"copies": nc, "ms_per_step": nn_ms,
                              "saved_us": round((nn_ms["block_then_inject_norm"] - nn_ms["block_next_norm"]) * 1e3, 1)}
        del hyper, mixed

    # The chunk report of the prefill.rs page (struct ChunkStats) for one
    # step: rows and expert-row statistics of the last step's grouping, the
    # records fetched over the host link (ring only), and the GPU time of the
    # experts' launches, from an extra pass with every phase timed by events
    # (per-launch durations; the events' own gaps stay out of `value`).
    cs = blk.chunk_stats()
    n_ph = steps if args.phases else min(steps, 10)
    mep.moe_profile_begin(mep.PHASES)
    for i in range(n_ph):
        step(i)
    torch.cuda.synchronize()
    ph = mep.moe_profile_end()
    expert_phases = ("shared_gateup", "shared_down", "gateup", "down", "experts", "combine")
    cs["secs"] = round(step_s, 7)
    cs["gpu_experts_s"] = round(sum(ph[p][0] for p in expert_phases if p in ph) / n_ph / 1e3, 7)
    extra["chunk_stats"] = cs
    if args.phases:
        extra["phase_us"] = {p: round(v[0] / v[1] * 1e3, 2) for p, v in ph.items()}
    res = dict(value=value, ms_per_step=ms_per_step, warmup=warmup, roofline=roofline, extra=extra,
               resident=int(resident.sum()) if resident is not None else cfg.experts)
    del blk, sets, pools
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def read_probe(reps: int = 5) -> dict:
    """The HBM read probe (moe_debug_read_probe): best of `reps` event-timed
    launches reading READ_PROBE_BYTES once, as the practical read ceiling the
    weight-streaming launches are compared with (the roofline keeps the
    published 8 TB/s as its peak)."""
    import torch

    import mixture_experts_prefill_amd as mep

    src = torch.ones(READ_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(READ_PROBE_BLOCKS, dtype=torch.int32, device="cuda")
    for _ in range(2):
        mep.moe_debug_read_probe(src, READ_PROBE_BLOCKS, sink)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        mep.moe_debug_read_probe(src, READ_PROBE_BLOCKS, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, sink
    torch.cuda.empty_cache()
    gbs = READ_PROBE_BYTES / (best / 1e3) / 1e9
    return {"kernel": "k_read_probe (16-byte non-temporal loads, grid-stride, 4 in flight per thread)",
            "bytes": READ_PROBE_BYTES, "blocks": READ_PROBE_BLOCKS, "best_ms": round(best, 4),
            "GBps": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 20 and at least 30 ms of work)")
    ap.add_argument("--config", default="full")
    ap.add_argument("--all-resident", action="store_true",
                    help="large: every expert resident in HBM instead of the top 64 plus the ring")
    ap.add_argument("--miss-bits", type=int, default=4, choices=(4, 2),
                    help="large: code width of the streamed (non-resident) experts' records over the host link")
    ap.add_argument("--copies", type=int, default=0,
                    help="weight copies rotated per step (0: enough that a step's weights have left the "
                         "256 MB MALL before the same copy comes round again)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of the oracle CPU-baseline sample (0: skip)")
    ap.add_argument("--cpu-rows-1t", type=int, default=128,
                    help="rows of the single-threaded oracle sample (0: skip)")
    ap.add_argument("--decode-extra", type=int, default=1,
                    help="with the full chunk, also time the decode-shaped chunks (t = 8 and t = 1)")
    ap.add_argument("--next-norm-copies", type=int, default=4,
                    help="residual copies of the next-norm timing leg (the block output injected into the next "
                         "fused norm, fused against separate calls); 0 skips it")
    ap.add_argument("--phases", action="store_true", help="also time every phase in an extra pass")
    ap.add_argument("--time-every", type=int, default=5,
                    help="time the dominant kernel's launch with HIP events in every N-th timed step")
    ap.add_argument("--separate", action="store_true",
                    help="run the shared expert as its own call (moe_shared) instead of inside the routed launches")
    ap.add_argument("--read-probe", type=int, default=1,
                    help="also time the HBM read probe (the device's practical read ceiling); 0 skips it")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy 512 MiB device-to-device (calibrates HBM byte counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files into profiles/traffic.json")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc, config=args.config, separate=args.separate)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the block is built and measured "
              f"on a single MI355X, with no sharding or collectives.", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_synth as ms

    torch.cuda.set_device(0)
    cfg = ms.CONFIGS[args.config]
    res = measure(cfg, args, args.steps, args.warmup, all_resident=args.all_resident, separate=args.separate)
    extra = res["extra"]
    if args.config == "full" and args.decode_extra and not args.separate:
        # The decode-shaped chunks (the HBM-bound case), timed the same way.
        for name in ("decode", "decode1"):
            dc = ms.CONFIGS[name]
            d = measure(dc, args, max(args.steps, 50), args.warmup)
            extra[f"{name}_t{dc.t}"] = {
                "ms_per_step": round(d["ms_per_step"], 4), "tokens_per_s": round(d["value"], 1),
                "block_hbm_frac": d["extra"]["block_hbm_frac"],
                "block_algorithmic_bytes": d["extra"]["block_algorithmic_bytes"],
                "touched_experts": d["extra"]["touched_experts"], "weight_copies": d["extra"]["weight_copies"],
                "warmup": d["warmup"], "step_ms_p10_p50_p90": d["extra"]["step_ms_p10_p50_p90"],
                "roofline": d["roofline"], "next_norm": d["extra"].get("next_norm"),
                "chunk_stats": d["extra"]["chunk_stats"]}

    if args.read_probe:
        # The practical read ceiling of this device, for the HBM-bound rows.
        probe = read_probe()
        extra["hbm_read_probe"] = probe
        for key in ("decode_t8", "decode1_t1"):
            if key in extra:
                d = extra[key]
                d["block_frac_of_read_probe"] = round(d["block_hbm_frac"] * PEAK_HBM_GBS / probe["GBps"], 4)
                if d["roofline"]["bound"] == "hbm":
                    d["roofline"]["frac_of_read_probe"] = round(d["roofline"]["achieved"] / probe["GBps"], 4)

    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_rows > 0:
        log(f"[bench] oracle CPU baseline on {args.cpu_rows} rows (+{args.cpu_rows_1t} single-threaded) ...")
        cpu = cpu_baseline(cfg.name, min(args.cpu_rows, cfg.t), min(args.cpu_rows_1t, cfg.t))

    workload = f"{cfg.name}: {cfg.description}"
    if args.all_resident and cfg.resident:
        workload += " (here every expert resident in HBM)"
    elif cfg.resident and args.miss_bits == 2:
        workload += " (streamed experts as 2-bit records, expanded on the GPU)"
    line = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": res["warmup"], "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "t": cfg.t, "hidden": cfg.hidden, "inter": cfg.inter,
                   "inter_shared": cfg.inter_shared, "experts": cfg.experts, "top_k": cfg.k, "group": cfg.group,
                   "weights": "int4 + fp16 scale/bias per group", "zipf_s": cfg.zipf_s,
                   "resident_experts": res["resident"], "parallelism": "none (1 GPU)"},
        "roofline": res["roofline"], "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
