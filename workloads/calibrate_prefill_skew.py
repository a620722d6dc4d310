"""Find the router-row skew exponent gamma of the prefill workload.

Writes ``prefill_router_skew.json``.  The target is the one the workload
names: expert popularity following Zipf(s=1.1).  A literal Zipf over 65,536
(token, expert) assignments cannot be realised because a token picks an expert
at most once (the first rank would need ~20 % of all assignments, more than
the 8,192 tokens), so the skew is fitted instead: gamma is bisected until the
log-log slope of the sorted non-zero per-expert counts over ranks 1..32 is
-1.1.  Routing here uses the CPU oracle's router on the seeded tokens.

Run from the repository root:  python -m workloads.calibrate_prefill_skew
"""

import json
import os

import numpy as np

import workloads as W
from oracle.route import route

TARGET_SLOPE = -1.1


def slope_for(gamma, x):
    cfg = W.PREFILL
    wr = W.router_weights(cfg, gamma=gamma)
    ids, _, _, _ = route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
    cnt = np.bincount(ids.ravel(), minlength=cfg.E)
    nz = np.sort(cnt[cnt > 0])[::-1][:32]
    s = np.polyfit(np.log(np.arange(1, len(nz) + 1)), np.log(nz), 1)[0]
    return float(s), cnt


def main():
    x = W.activations(W.PREFILL)
    lo, hi = 1.0, 6.0
    for _ in range(12):
        mid = 0.5 * (lo + hi)
        s, _ = slope_for(mid, x)
        print(f"gamma={mid:.5f} slope={s:.4f}", flush=True)
        if s > TARGET_SLOPE:
            lo = mid
        else:
            hi = mid
    gamma = round(0.5 * (lo + hi), 4)
    s, cnt = slope_for(gamma, x)
    out = {
        "gamma": gamma,
        "c_max": W.C_MAX,
        "slope_ranks_1_32": round(s, 4),
        "experts_over_1000": int((cnt > 1000).sum()),
        "experts_0_to_8": int((cnt <= 8).sum()),
        "experts_zero": int((cnt == 0).sum()),
        "max_count": int(cnt.max()),
        "_comment": "written by workloads/calibrate_prefill_skew.py (routes the seeded prefill tokens with the CPU oracle)",
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "prefill_router_skew.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
