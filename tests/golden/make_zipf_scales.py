"""Fit the Zipf bias strength s for every (workload, imbalance target).

Writes tests/golden/zipf_scales.json.  The imbalance of a candidate routing is
measured with the oracle's maxvio only; the routing itself comes from the
seeded generator.  Bisection on s until |maxvio - target| <= 0.05 (or the
closest point after 40 steps).  Run from the repository root:

    python tests/golden/make_zipf_scales.py
"""
import json
import os
import sys

_REPO = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, _REPO)

import moonep_synth as synth  # noqa: E402
import oracle  # noqa: E402


def fit(w, target, seed=0):
    lo, hi = 0.0, 8.0
    best = None
    for _ in range(40):
        s = 0.5 * (lo + hi)
        topk, _ = synth.routing_zipf(w, s, seed)
        mv = oracle.maxvio(topk, w.E)
        if best is None or abs(mv - target) < abs(best[1] - target):
            best = (s, mv)
        if abs(mv - target) <= 0.05:
            break
        if mv < target:
            lo = s
        else:
            hi = s
    return best


def main():
    table = {}
    for name, targets in synth.SWEEPS.items():
        w = synth.WORKLOADS[name]
        table[name] = {}
        for t in targets:
            if t == "adv" or float(t) == 0.0:
                continue
            s, mv = fit(w, float(t))
            table[name][str(float(t))] = s
            print(f"{name} target={t} s={s:.6f} maxvio={mv:.4f}", flush=True)
    with open(synth.ZIPF_TABLE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
