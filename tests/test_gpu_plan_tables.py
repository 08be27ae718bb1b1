"""The derived tables moonep_plan writes into plan.aux, against what the
oracle plan implies: each rank's active rows, the used prefetch slots, the
reduce_grad holder tables (README "Gradient buffer": the prefetch-slot
gradients of every holder of a home expert, added in ascending rank), and the
grouped-GEMM M-tile schedule (every padded row of every segment in exactly one
tile of at most 256 rows that never crosses a segment, full-height tiles
first).  The offsets follow the AuxLayout the library documents for aux
(act, pf_n, pf, dup_n, dup_e, dup_first, dup_cnt, hold, tiles, ntiles, nfull,
nact, in that order)."""
import numpy as np
import pytest

import moonep_synth as synth
import oracle
from gpu_util import buffer_for, dev, log, plan_host
from test_gpu_planning import EDGE

pytestmark = pytest.mark.gpu


def aux_layout(w, NvS):
    R, E, B = w.R, w.E, w.B
    L = E // R
    RB = R * B
    o = {"act": 0}
    o["pf_n"] = o["act"] + 2 * E
    o["pf"] = o["pf_n"] + 1
    o["dup_n"] = o["pf"] + RB
    o["dup_e"] = o["dup_n"] + 1
    o["dup_first"] = o["dup_e"] + RB
    o["dup_cnt"] = o["dup_first"] + RB
    o["hold"] = o["dup_cnt"] + RB
    max_tiles = -(-NvS // 256) + 2 * L
    o["tiles"] = o["hold"] + RB
    o["ntiles"] = o["tiles"] + 4 * R * max_tiles
    o["nfull"] = o["ntiles"] + R
    o["nact"] = o["nfull"] + R
    return o, max_tiles


def expected_tables(w, p):
    """act/nact, the used prefetch slots and the holder tables, from the
    oracle plan's public arrays."""
    R, E, B = w.R, w.E, w.B
    L2 = 2 * (E // R)
    act = np.full((R, L2), -1, np.int64)
    nact = np.zeros(R, np.int64)
    for d in range(R):
        rows = np.nonzero(p.seg_tokens[d] > 0)[0]
        act[d, :len(rows)] = rows
        nact[d] = len(rows)
    pf = p.prefetch_src.reshape(R, B)
    used = [d * B + j for d in range(R) for j in range(B) if pf[d, j] >= 0]
    dup_e, dup_first, dup_cnt, hold = [], [], [], []
    for e in range(E):
        holders = [d * B + j for d in range(R) for j in range(B) if pf[d, j] == e]
        if holders:
            dup_e.append(e)
            dup_first.append(len(hold))
            dup_cnt.append(len(holders))
            hold += holders
    return act, nact, used, dup_e, dup_first, dup_cnt, hold


def check_tiles(w, p, tiles, ntiles, nfull):
    """Every padded row of every segment lies in exactly one tile; a tile has
    at most 256 rows of one segment and names its row; tiles of more than
    128 rows (or whole 256-row ones) come first, the <=128-row segment tails
    after them; group fields name a run of tiles of one segment."""
    R, E, B, tp = w.R, w.E, w.B, w.token_padding
    for d in range(R):
        n, nf = int(ntiles[d]), int(nfull[d])
        t = tiles[d, :n]
        cover = {}
        for row in range(E + B):
            cnt = int(p.seg_tokens[d, row])
            if cnt == 0:
                continue
            end = int(p.cu_seqlens[d, row])
            ln = -(-cnt // tp) * tp
            cover[row] = (end - ln, end)
        seen = {row: [] for row in cover}
        for i, (row, m0, m1, grp) in enumerate(t):
            assert row in cover, f"rank {d} tile {i}: row {row} is not active"
            lo, hi = cover[row]
            assert lo <= m0 < m1 <= hi and m1 - m0 <= 256, f"rank {d} tile {i}"
            seen[row].append((m0, m1))
            if i < nf:
                assert m1 - m0 > 128, f"rank {d} tile {i}: a short tile among the full ones"
            else:
                assert m1 - m0 <= 128, f"rank {d} tile {i}: a full tile after the short ones"
            gs, gm = grp >> 4, grp & 15
            assert gs <= i < gs + gm and 1 <= gm <= 8
        for row, (lo, hi) in cover.items():
            pieces = sorted(seen[row])
            assert pieces and pieces[0][0] == lo and pieces[-1][1] == hi, f"rank {d} row {row}"
            for (a0, a1), (b0, b1) in zip(pieces, pieces[1:]):
                assert a1 == b0, f"rank {d} row {row}: gap or overlap at {a1}"


def run_tables(w, topk, buf=None):
    log(f"plan tables {w.name} R={w.R} S={w.S} K={w.K} E={w.E} B={w.B} tp={w.token_padding}")
    own = buf is None
    buf = buffer_for(w) if own else buf
    plan = buf.plan(dev(topk))
    got = plan_host(buf, plan)
    aux = plan.arrays["aux"].cpu().numpy()
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    assert got["stats"][0] == 0
    assert np.array_equal(got["cu_seqlens"], p.cu_seqlens)
    assert np.array_equal(got["seg_tokens"], p.seg_tokens)
    o, max_tiles = aux_layout(w, buf.NvS)
    R, RB, L2 = w.R, w.R * w.B, 2 * (w.E // w.R)
    act, nact, used, dup_e, dup_first, dup_cnt, hold = expected_tables(w, p)
    assert np.array_equal(aux[o["act"]:o["act"] + R * L2].reshape(R, L2), act)
    assert np.array_equal(aux[o["nact"]:o["nact"] + R], nact)
    assert aux[o["pf_n"]] == len(used)
    assert list(aux[o["pf"]:o["pf"] + len(used)]) == used
    nd = int(aux[o["dup_n"]])
    assert nd == len(dup_e)
    assert list(aux[o["dup_e"]:o["dup_e"] + nd]) == dup_e
    assert list(aux[o["dup_first"]:o["dup_first"] + nd]) == dup_first
    assert list(aux[o["dup_cnt"]:o["dup_cnt"] + nd]) == dup_cnt
    assert list(aux[o["hold"]:o["hold"] + len(hold)]) == hold
    tiles = aux[o["tiles"]:o["tiles"] + 4 * R * max_tiles].reshape(R, max_tiles, 4)
    check_tiles(w, p, tiles, aux[o["ntiles"]:o["ntiles"] + R], aux[o["nfull"]:o["nfull"] + R])
    if own:
        buf.destroy()


@pytest.mark.parametrize("name,target", [
    ("tiny_r4_s64_k2_e8", 0.0), ("tiny_r4_s64_k2_e8", 1.0), ("mid_r8_s1024_k4_e32", 0.0),
    ("mid_r8_s1024_k4_e32", 1.0), ("mid_r8_s1024_k4_e32", 2.0), ("fwd_r8_s4096_k8_e256", 0.0),
    ("fwd_r8_s4096_k8_e256", 2.0), ("fwd_r8_s4096_k8_e256", "adv"),
    ("infer_r8_s128_k8_e256_b4", 4.0)])
def test_plan_tables(name, target):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing(w, target)
    run_tables(w, topk)


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
def test_plan_tables_edge_shapes(w):
    topk, _ = synth.routing_zipf(w, 1.5, seed=7)
    run_tables(w, topk)


def test_plan_tables_after_failed_plan():
    """A plan of bad routing leaves no segment, no prefetch, no holder and no
    tile; a good plan on the same handle afterwards is whole again."""
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    topk, _ = synth.routing(w, 2.0)
    bad = topk.copy()
    bad[0, 0, 0] = w.E
    buf = buffer_for(w)
    plan = buf.plan(dev(bad))
    got = plan_host(buf, plan)
    aux = plan.arrays["aux"].cpu().numpy()
    o, _ = aux_layout(w, buf.NvS)
    assert got["stats"][0] & 1
    assert aux[o["pf_n"]] == 0 and aux[o["dup_n"]] == 0
    assert (aux[o["ntiles"]:o["ntiles"] + w.R] == 0).all()
    assert (aux[o["nact"]:o["nact"] + w.R] == 0).all()
    run_tables(w, topk, buf)
    buf.destroy()
