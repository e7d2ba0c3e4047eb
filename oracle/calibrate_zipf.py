"""Choose the router-row gain exponent alpha of the Zipf-skewed workloads.

Workload recipe (not part of the method): router row e is scaled by
(pi(e)+1)^-alpha for a seeded permutation pi.  alpha is picked on the grid
0.00:0.01:1.00 so that the least-squares slope of log(rows per expert) against
log(popularity rank), over non-empty experts, is closest to -s.  The grid
search uses float64 logits (gain times the unscaled logits) to rank quickly;
the chosen alpha is then re-checked with the oracle's own fp32 router and
top-k, and that realised histogram is what gets stored.

Writes moe_synth/zipf_alpha.json.  Run: python oracle/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import moe_synth as ms  # noqa: E402
import oracle  # noqa: E402


def slope(counts):
    c = np.sort(counts[counts > 0])[::-1].astype(np.float64)
    r = np.arange(1, c.size + 1, dtype=np.float64)
    A = np.stack([np.log(r), np.ones_like(r)], 1)
    return float(np.linalg.lstsq(A, np.log(c), rcond=None)[0][0])


def counts_from_topk(idx, E):
    return np.bincount(idx.reshape(-1), minlength=E)


def calibrate(name):
    cfg = ms.CONFIGS[name]
    x = ms.bf16_bits_to_f32(ms.make_x(cfg)).astype(np.float64)
    w0 = ms.make_router(cfg, alpha=0.0).astype(np.float64)
    base = x @ w0.T
    best = None
    for a in np.round(np.arange(0.0, 1.0001, 0.01), 2):
        lg = base * ms.zipf_gain(cfg, a)[None, :]
        idx = np.argsort(-lg, axis=1, kind="stable")[:, :cfg.k]
        s = slope(counts_from_topk(idx, cfg.experts))
        if best is None or abs(s + cfg.zipf_s) < best[1]:
            best = (float(a), abs(s + cfg.zipf_s), s)
    alpha = best[0]
    lg = oracle.router_logits(ms.make_x(cfg), ms.make_router(cfg, alpha))
    idx, _ = oracle.topk(lg, cfg.k)
    c = counts_from_topk(idx, cfg.experts)
    return {"alpha": alpha, "target_s": cfg.zipf_s, "slope": round(slope(c), 4),
            "max_rows": int(c.max()), "median_rows": float(np.median(c)),
            "nonempty": int((c > 0).sum()), "experts": cfg.experts}


if __name__ == "__main__":
    out = {n: calibrate(n) for n in ("full", "large")}
    with open(os.path.join(ROOT, "moe_synth", "zipf_alpha.json"), "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(out, indent=2))
