"""The benchmark's algorithmic work (bench.algorithmic), which the roofline
figures divide by measured time, against closed forms worked out by hand
from the workload shapes (one record = 3 h I (1/2 + 4/G) bytes: int4 codes
and an fp16 scale and bias per group; gate and up are two thirds of it).
"""
import numpy as np

import bench
import moe_synth as ms


def test_full_chunk_merged_launch():
    cfg = ms.CONFIGS["full"]                      # t 4096, h 2048, I 768, E 128, k 8, G 64, shared I 768
    w = bench.algorithmic(cfg, cfg.t, np.ones(cfg.experts), fused=True)
    gu_rec, dn_rec = 1_769_472, 884_736           # 2/3 and 1/3 of 2,654,208
    rows = 4096 * 8 + 4096                        # CSR rows plus the shared expert's rows
    gateup = 129 * gu_rec + 4096 * 2048 * 2 + rows * 768 * 2
    down = 129 * dn_rec + rows * 768 * 2 + rows * 2048 * 2
    assert w["bytes_gateup"] == gateup == 301_662_208
    assert w["bytes_down"] == down == 321_748_992
    assert w["flop_gateup"] + w["flop_down"] == 6 * 4096 * 2048 * (8 * 768 + 768) == 347_892_350_976
    assert w["flop_shared"] == 0                  # counted inside the merged launch


def test_decode_chunk_merged_launch():
    cfg = ms.CONFIGS["decode"]                    # t 8, h 4096, I 1536, E 512, k 10, G 64
    counts = np.zeros(cfg.experts)
    counts[:74] = 1                               # 74 touched experts
    w = bench.algorithmic(cfg, cfg.t, counts, fused=True)
    gu_rec, dn_rec = 7_077_888, 3_538_944         # 2/3 and 1/3 of 10,616,832
    rows = 8 * 10 + 8
    assert w["bytes_gateup"] + w["bytes_down"] == (75 * (gu_rec + dn_rec) + 8 * 4096 * 2 + 2 * rows * 1536 * 2
                                                  + rows * 4096 * 2) == 797_589_504
    # the whole block: every touched record and the shared one, the fp32 router weights, x and out
    assert w["bytes_total"] == 74 * 10_616_832 + 10_616_832 + 4 * 512 * 4096 + 2 * 8 * 4096 + 4 * 8 * 4096


def test_separate_calls_count_no_shared_rows():
    cfg = ms.CONFIGS["full"]
    w = bench.algorithmic(cfg, cfg.t, np.ones(cfg.experts), fused=False)
    assert w["flop_gateup"] == 4 * 4096 * 8 * 2048 * 768
    assert w["flop_down"] == 2 * 4096 * 8 * 2048 * 768
    assert w["flop_shared"] == 6 * 4096 * 2048 * 768
