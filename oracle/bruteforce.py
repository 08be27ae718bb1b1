"""Exact minimum number of redundant experts, by enumeration.
TEST INFRASTRUCTURE ONLY; tiny inputs only.

A placement gives every rank exactly C = S*K slots (MoonEP README item 1),
takes every token of every expert, and lets a rank hold, besides its own home
experts, experts of at most one remote home group (README "How to set B").
A redundant expert is a (rank, remote expert) pair with at least one token.
Only the expert loads T_e matter for the count, so the search is over which
remote experts each rank may hold; feasibility of a choice is a max-flow
problem (source -> expert with capacity T_e, expert -> allowed rank, rank ->
sink with capacity C), solved with scipy's maximum_flow.
"""
import itertools

import numpy as np
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import maximum_flow


def _feasible(T, R, L, C, allowed):
    E = len(T)
    n = 2 + E + R
    src, sink = 0, n - 1
    rows, cols, caps = [], [], []
    for e in range(E):
        if T[e]:
            rows.append(src); cols.append(1 + e); caps.append(int(T[e]))
            rows.append(1 + e); cols.append(1 + E + e // L); caps.append(int(C))
    for (d, e) in allowed:
        rows.append(1 + e); cols.append(1 + E + d); caps.append(int(C))
    for d in range(R):
        rows.append(1 + E + d); cols.append(sink); caps.append(int(C))
    m = csr_matrix((np.array(caps, dtype=np.int32), (rows, cols)), shape=(n, n))
    return maximum_flow(m, src, sink).flow_value == int(sum(T))


def min_duplicates(T, R: int, C: int, max_k=None) -> int:
    """Smallest number of (rank, remote expert) pairs of any valid placement."""
    T = [int(t) for t in T]
    E = len(T)
    L = E // R
    assert sum(T) == R * C
    # per rank: None, or (remote group, non-empty subset of its loaded experts)
    options = []
    for d in range(R):
        opts = [()]
        for g in range(R):
            if g == d:
                continue
            loaded = [e for e in range(g * L, (g + 1) * L) if T[e] > 0]
            for size in range(1, len(loaded) + 1):
                opts.extend(itertools.combinations(loaded, size))
        options.append(opts)
    limit = max_k if max_k is not None else R * L
    for k in range(0, limit + 1):
        # choices whose subset sizes add up to exactly k
        def rec(d, left, chosen):
            if d == R:
                if left == 0:
                    allowed = [(dd, e) for dd, sub in enumerate(chosen) for e in sub]
                    if _feasible(T, R, L, C, allowed):
                        return True
                return False
            for sub in options[d]:
                if len(sub) <= left and rec(d + 1, left - len(sub), chosen + [sub]):
                    return True
            return False
        if rec(0, k, []):
            return k
    raise RuntimeError("no placement found")
