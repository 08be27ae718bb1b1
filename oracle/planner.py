"""Balanced redundant-expert planner (spec P1-P9).  TEST INFRASTRUCTURE ONLY.

What the pages fix (MoonEP README, items 1-2, "Usage > Integration",
"Weight buffer", "How to set B", "API guide > dispatch fwd"; MarkTechPost
article, sections "The core idea" and "Memory contract"):

* every EP rank receives exactly S*K token-slots, however skewed the routing;
* a rank duplicates experts from at most one remote home group (<= E/R
  experts), so training works with B = E/R prefetch slots;
* dispatched tokens sit in expert-grouped order; cu_seqlens[E+B] holds the
  padded end offset of each row of the [E+B,H,H'] weight tensor; rows [0,E)
  are home experts (E/R per rank), rows [E,E+B) local prefetch slots; remote
  experts beyond B are read from their home rows [0,E).

The pages call the planner "near-optimal" but do not print it.  This module
is the spec the GPU planner must reproduce bit for bit:

P1  c[r][e] = slots of rank r on expert e;  T_e = sum_r c[r][e].
P2  group load W_g = sum of T_e over the L = E/R experts homed on rank g.
P3  keep_g = min(W_g, C), excess X_g = W_g - keep_g, deficit D_g = C - keep_g,
    where C = S*K.
P4  donors: groups with X_g > 0, ordered by (-X_g, g); receiver queue: ranks
    with D_r > 0, ordered by (-D_r, r); need[r] = D_r.
P5  chain-greedy: the current donor gives each receiver popped from the queue
    its whole need.  If the donor's remaining excess x is smaller than that
    need, the donor gives it anyway, shrinks its own keep by the shortfall,
    becomes a receiver of that shortfall at the back of the queue, and the
    next donor takes over.  Every rank ends up receiving at most one donation,
    from one group, and holding exactly C slots.
P6  the line of group g lists its experts by (T_e, e) ascending; expert e
    occupies [a_e, a_e + T_e).  The line is cut into pieces: [0, keep_g) to
    rank g, then g's donations in emission order, back to back.
P7  the tokens of expert e are ordered by (r, s); the line position of (r,s,k)
    is a_e + sum_{r'<r} c[r'][e] + #{s' < s on rank r routed to e}.  The
    piece holding that position names the destination rank d.
P8  rows on d: a home expert (e // L == d) uses row e; remote experts, in
    ascending e, use rows E, E+1, ... while j < B (prefetch_src[d][j] = e)
    and their home row e beyond that (overflow, only when B < E/R).
P9  len = round_up(n, token_padding) per row (0 stays 0); cu_seqlens is the
    inclusive prefix sum of len over the E+B rows; the slot of a token is
    cu_seqlens[row] - len[row] + (position - start of (d, e)'s range).
"""
from __future__ import annotations

import dataclasses
from collections import deque

import numpy as np


def nvs(S: int, K: int, E: int, R: int, token_padding: int) -> int:
    """Token slots per rank: S*K real ones plus the padding of at most 2*E/R
    active rows (E/R home rows and at most E/R rows of one remote group), each
    padded by less than token_padding.  The README's notation ("Usage >
    Integration") defines NvS only as the S*K real slots plus per-row padding;
    this bound is the smallest size that fits every plan P1-P9 can make."""
    return S * K + 2 * (E // R) * token_padding


def round_up(n: int, m: int) -> int:
    return ((n + m - 1) // m) * m


@dataclasses.dataclass
class Plan:
    R: int
    S: int
    K: int
    E: int
    B: int
    tp: int
    NvS: int
    counts: np.ndarray          # [R,E]  c[r][e]
    T: np.ndarray               # [E]
    W: np.ndarray               # [R]   group loads
    keep: np.ndarray            # [R]   final home keep
    donations: list             # [(g, r, amount)] in emission order
    line_start: np.ndarray      # [E]   a_e
    pieces: list                # per group: [(lo, hi, rank)]
    remote_group: np.ndarray    # [R]   -1 if none
    remote_experts: list        # per rank: sorted expert ids
    prefetch_src: np.ndarray    # [R,B] -1 unused
    row_of: list                # per rank: {expert: row}
    seg_tokens: np.ndarray      # [R,E+B] real tokens per row
    seg_len: np.ndarray         # [R,E+B] padded length per row
    cu_seqlens: np.ndarray      # [R,E+B] inclusive padded end offsets
    dest: np.ndarray            # [R,S,K] d*NvS + slot
    src: np.ndarray             # [R,NvS] (r*S+s)*K+k, -1 = no token
    dup_count: int

    @property
    def L(self):
        return self.E // self.R

    @property
    def C(self):
        return self.S * self.K


def _donations(R: int, C: int, W: np.ndarray):
    """P3-P5: keeps and the chain-greedy donation list."""
    keep = np.minimum(W, C).astype(np.int64)
    X = W - keep
    D = C - keep
    donors = sorted([g for g in range(R) if X[g] > 0], key=lambda g: (-X[g], g))
    queue = deque(sorted([r for r in range(R) if D[r] > 0], key=lambda r: (-D[r], r)))
    need = D.astype(np.int64).copy()
    out = []
    if not donors:
        assert not queue
        return keep, out
    i = 0
    x = int(X[donors[0]])
    while queue:
        r = queue.popleft()
        d = int(need[r])
        g = donors[i]
        out.append((g, r, d))
        if d <= x:
            x -= d
            if x == 0 and i + 1 < len(donors):
                i += 1
                x = int(X[donors[i]])
        else:
            short = d - x
            keep[g] -= short
            need[g] = short
            queue.append(g)
            i += 1
            x = int(X[donors[i]])
    return keep, out


def plan(topk: np.ndarray, E: int, B: int, token_padding: int) -> Plan:
    topk = np.asarray(topk, dtype=np.int64)
    R, S, K = topk.shape
    if E % R:
        raise ValueError("E must be a multiple of R")
    L = E // R
    C = S * K
    tp = token_padding
    NvS = nvs(S, K, E, R, tp)
    if topk.min(initial=0) < 0 or topk.max(initial=0) >= E:
        raise ValueError("expert id out of range")
    for r in range(R):
        for s in range(S):
            if len(set(topk[r, s].tolist())) != K:
                raise ValueError("repeated expert id within a token")

    # P1
    counts = np.zeros((R, E), dtype=np.int64)
    for r in range(R):
        for e in topk[r].reshape(-1).tolist():
            counts[r, e] += 1
    T = counts.sum(axis=0)
    # P2
    W = np.array([T[g * L:(g + 1) * L].sum() for g in range(R)], dtype=np.int64)
    # P3-P5
    keep, donations = _donations(R, C, W)

    # P6: lines and pieces
    line_start = np.zeros(E, dtype=np.int64)
    for g in range(R):
        experts = sorted(range(g * L, (g + 1) * L), key=lambda e: (T[e], e))
        a = 0
        for e in experts:
            line_start[e] = a
            a += T[e]
    pieces = []
    for g in range(R):
        ps = []
        lo = 0
        if keep[g] > 0:
            ps.append((0, int(keep[g]), g))
            lo = int(keep[g])
        for (dg, r, amount) in donations:
            if dg == g:
                ps.append((lo, lo + amount, r))
                lo += amount
        assert lo == W[g]
        pieces.append(ps)

    # tokens of each expert held by each rank: overlap of the expert's range
    # with the rank's piece of that expert's group
    held = np.zeros((R, E), dtype=np.int64)        # n for (d, e)
    range_lo = np.full((R, E), -1, dtype=np.int64)  # first line position of (d,e)
    for e in range(E):
        g = e // L
        a0, a1 = line_start[e], line_start[e] + T[e]
        for (lo, hi, d) in pieces[g]:
            n = min(a1, hi) - max(a0, lo)
            if n > 0:
                held[d, e] = n
                range_lo[d, e] = max(a0, lo)

    # P8: rows
    remote_group = np.full(R, -1, dtype=np.int64)
    remote_experts = []
    prefetch_src = np.full((R, B), -1, dtype=np.int64)
    row_of = []
    for d in range(R):
        rows = {}
        rem = []
        for e in range(E):
            if held[d, e] == 0:
                continue
            if e // L == d:
                rows[e] = e
            else:
                rem.append(e)
        groups = {e // L for e in rem}
        assert len(groups) <= 1
        if rem:
            remote_group[d] = rem[0] // L
        for j, e in enumerate(rem):
            if j < B:
                rows[e] = E + j
                prefetch_src[d, j] = e
            else:
                rows[e] = e
        remote_experts.append(rem)
        row_of.append(rows)

    # P9: lengths and cu_seqlens
    seg_tokens = np.zeros((R, E + B), dtype=np.int64)
    for d in range(R):
        for e, row in row_of[d].items():
            seg_tokens[d, row] = held[d, e]
    seg_len = np.array([[round_up(int(n), tp) for n in row] for row in seg_tokens],
                       dtype=np.int64).reshape(R, E + B)
    cu_seqlens = np.cumsum(seg_len, axis=1)
    assert (cu_seqlens[:, -1] <= NvS).all()

    # P7: destination of every (r, s, k)
    rank_before = np.cumsum(counts, axis=0) - counts   # sum_{r'<r} c[r'][e]
    dest = np.empty((R, S, K), dtype=np.int64)
    src = np.full((R, NvS), -1, dtype=np.int64)
    for r in range(R):
        seen = np.zeros(E, dtype=np.int64)
        for s in range(S):
            for k in range(K):
                e = int(topk[r, s, k])
                pos = line_start[e] + rank_before[r, e] + seen[e]
                seen[e] += 1
                d = next(pd for (lo, hi, pd) in pieces[e // L] if lo <= pos < hi)
                row = row_of[d][e]
                slot = cu_seqlens[d, row] - seg_len[d, row] + (pos - range_lo[d, e])
                dest[r, s, k] = d * NvS + slot
                src[d, slot] = (r * S + s) * K + k

    dup_count = int(sum(len(x) for x in remote_experts))
    return Plan(R=R, S=S, K=K, E=E, B=B, tp=tp, NvS=NvS, counts=counts, T=T,
                W=W, keep=keep, donations=donations, line_start=line_start,
                pieces=pieces, remote_group=remote_group,
                remote_experts=remote_experts, prefetch_src=prefetch_src,
                row_of=row_of, seg_tokens=seg_tokens, seg_len=seg_len,
                cu_seqlens=cu_seqlens, dest=dest, src=src, dup_count=dup_count)
