"""Properties every valid plan has, whoever computed it.

Used to pin the oracle's planner (tests/test_oracle_planner.py) and to check
GPU plans at sizes where the oracle is not run in full.  Sources: MoonEP
README item 1 (exactly S*K slots per rank), "How to set B" (at most one
remote home group per rank; with B = E/R every remote expert is local),
"API guide > dispatch fwd" (expert-grouped rows, padded end offsets).
"""
import numpy as np


def round_up(n, m):
    return (n + m - 1) // m * m


def check_plan_arrays(topk, E, B, tp, NvS, dest, src, cu_seqlens, seg_tokens,
                      prefetch_src):
    """Check a plan given as plain arrays; raises AssertionError on a defect.
    dest [R,S,K] global slots, src [R,NvS], cu_seqlens / seg_tokens [R,E+B],
    prefetch_src [R,B]."""
    topk = np.asarray(topk, dtype=np.int64)
    R, S, K = topk.shape
    L = E // R
    C = S * K
    dest = np.asarray(dest, dtype=np.int64)
    src = np.asarray(src, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nt = np.asarray(seg_tokens, dtype=np.int64)
    pf = np.asarray(prefetch_src, dtype=np.int64)
    assert cu.shape == (R, E + B) and nt.shape == (R, E + B)

    # cu_seqlens: padded, monotone, inclusive, fits NvS
    ln = np.diff(np.concatenate([np.zeros((R, 1), np.int64), cu], axis=1), axis=1)
    assert (ln >= 0).all(), "cu_seqlens not monotone"
    assert (cu[:, -1] <= NvS).all(), "segments overflow NvS"
    assert (ln == round_up(nt, tp)).all(), "row length is not round_up(n, tp)"

    # every (r,s,k) lands exactly once; src inverts dest
    flat = dest.reshape(-1)
    assert flat.min() >= 0 and flat.max() < R * NvS
    assert np.unique(flat).size == flat.size, "two tokens share a slot"
    t = np.arange(R * S * K, dtype=np.int64)
    assert (src.reshape(-1)[flat] == t).all(), "src does not invert dest"
    assert (src >= 0).sum() == R * S * K

    # exactly S*K real slots on every rank
    assert ((src >= 0).sum(axis=1) == C).all(), "a rank does not get S*K slots"

    # prefetch table: used slots first, distinct experts
    for d in range(R):
        used = pf[d][pf[d] >= 0]
        assert (pf[d][: used.size] == used).all() and (pf[d][used.size:] == -1).all()
        assert np.unique(used).size == used.size

    # each row: tokens of its expert, contiguous from the row start, then
    # padding; order (r, s) ascending; padding holds no token
    remote_groups = [set() for _ in range(R)]
    for d in range(R):
        start = 0
        for row in range(E + B):
            end = cu[d, row]
            n = nt[d, row]
            if end > start:
                if row < E:
                    e = row
                    if e // L != d:
                        assert B < L, "overflow row although B == E/R"
                        assert pf[d, B - 1] >= 0 if B > 0 else True
                        remote_groups[d].add(e // L)
                else:
                    e = pf[d, row - E]
                    assert e >= 0, "segment in an unused prefetch row"
                    remote_groups[d].add(e // L)
                    assert e // L != d, "home expert in a prefetch row"
                seg = src[d, start:end]
                assert (seg[:n] >= 0).all() and (seg[n:] == -1).all()
                toks = seg[:n]
                r_, s_, k_ = toks // (S * K), (toks // K) % S, toks % K
                assert (topk[r_, s_, k_] == e).all(), "slot holds another expert"
                key = r_ * S + s_
                assert (np.diff(key) > 0).all(), "tokens not in (r, s) order"
            start = end
        assert (src[d, cu[d, -1]:] == -1).all()
    for d in range(R):
        assert len(remote_groups[d]) <= 1, "more than one remote home group"

    # each expert's tokens, in (r, s) order, form one contiguous run per rank
    for e in range(E):
        r_, s_, k_ = np.nonzero(topk == e)
        order = np.lexsort((s_, r_))
        d_seq = dest[r_[order], s_[order], k_[order]] // NvS
        if d_seq.size:
            changes = np.count_nonzero(np.diff(d_seq))
            assert changes == np.unique(d_seq).size - 1, "expert split non-contiguously"
    return True


def check_plan(p, topk):
    return check_plan_arrays(topk, p.E, p.B, p.tp, p.NvS, p.dest, p.src,
                             p.cu_seqlens, p.seg_tokens, p.prefetch_src)
