"""Seeded planner fuzz: moonep_plan on random shapes (R up to 8, up to 16
experts per rank, K up to 8, S up to 600, any B <= E/R, token_padding from 1 to
200) under random routing families -- Zipf popularity of random strength,
every rank sending to the next rank's experts, hot experts present in every
token, all tokens on the first K experts, exact balance -- against the oracle
planner bit for bit (every plan array and the stats) and the derived tables
against the oracle plan.  Shapes stay small so the oracle plans each in well
under a second."""
import numpy as np
import pytest

import moonep_synth as synth
from test_gpu_plan_tables import run_tables
from test_gpu_planning import run_and_compare

pytestmark = pytest.mark.gpu

CASES = 120
STREAM_CASE = 9         # sub-stream of the case generator (input draws only)


def fuzz_case(i):
    g = synth.rng(1000 + i, STREAM_CASE)
    R = int(g.choice([1, 2, 3, 4, 8]))
    L = int(g.integers(1, 17))
    E = R * L
    K = int(g.integers(1, min(E, 8) + 1))
    S = int(g.integers(1, 601))
    B = int(g.integers(0, L + 1))
    tp = int(g.choice([1, 2, 16, 64, 128, 200]))
    w = synth.Workload(f"fuzz{i}", R=R, S=S, K=K, E=E, B=B, H=64, Hp=64, token_padding=tp)
    kind = i % 5
    if kind == 0:
        s = float(g.uniform(0.0, 3.0))
        topk, _ = synth.routing_zipf(w, s, seed=i)
        desc = f"zipf s={s:.2f}"
    elif kind == 1:
        st = float(g.uniform(0.5, 4.0))
        topk, _ = synth.routing_rank_skew(w, st, seed=i)
        desc = f"rank-skew {st:.2f}"
    elif kind == 2:
        nhot = int(g.integers(1, K + 1))
        topk, _ = synth.routing_hot(w, nhot, seed=i)
        desc = f"hot {nhot}"
    elif kind == 3:
        topk, _ = synth.routing_adversarial(w, seed=i)
        desc = "adversarial"
    elif (R * S * K) % E == 0:
        topk, _ = synth.routing_balanced(w, seed=i)
        desc = "balanced"
    else:
        topk, _ = synth.routing_zipf(w, 1.0, seed=i)
        desc = "zipf s=1"
    return w, topk, desc


@pytest.mark.parametrize("i", range(CASES))
def test_plan_fuzz(i):
    w, topk, desc = fuzz_case(i)
    print(f"[fuzz] case {i}: {desc}", flush=True)
    run_and_compare(w, topk)
    run_tables(w, topk)
