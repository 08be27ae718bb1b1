"""Pins for the oracle's maxvio and planner.

* maxvio: closed forms (balanced routing -> 0, all tokens on experts
  0..K-1 -> E/K - 1, a hand case).
* planner: two hand-worked plans (one with a donation chain), closed forms for
  balanced and adversarial routing, the structural invariants the pages fix
  (exactly S*K slots per rank, every token-slot once, <= 1 remote home group,
  contiguous expert segments, padded cu_seqlens) on every workload and many
  random instances, and brute-force optima on tiny inputs.
"""
import numpy as np
import pytest

import moonep_synth as synth
import oracle
from oracle.planner import round_up
from plan_checks import check_plan


def topk_from_counts(count_lists, S, K):
    """Build a [R,S,K] routing whose per-rank expert counts are given, with
    distinct experts per token when K > 1 (only K == 1 used here)."""
    assert K == 1
    R = len(count_lists)
    topk = np.zeros((R, S, K), dtype=np.int32)
    for r, counts in enumerate(count_lists):
        ids = [e for e, c in enumerate(counts) for _ in range(c)]
        assert len(ids) == S
        topk[r, :, 0] = ids
    return topk


# ---------------------------------------------------------------- maxvio
def test_maxvio_hand_case():
    topk = np.array([[[0], [0]]], dtype=np.int32)      # R=1,S=2,K=1,E=2
    assert oracle.maxvio(topk, 2) == 1.0               # T=[2,0], T_bar=1


@pytest.mark.parametrize("name", ["tiny_r4_s64_k2_e8", "mid_r8_s1024_k4_e32",
                                  "fwd_r8_s4096_k8_e256"])
def test_maxvio_balanced_and_adversarial(name):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing_balanced(w)
    assert oracle.maxvio(topk, w.E) == 0.0
    topk, _ = synth.routing_adversarial(w)
    assert oracle.maxvio(topk, w.E) == pytest.approx(w.E / w.K - 1, abs=0)


def test_maxvio_headline_adversarial_is_31():
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    topk, _ = synth.routing_adversarial(w)
    assert oracle.maxvio(topk, w.E) == 31.0


# ---------------------------------------------------------- hand-worked
def test_hand_plan_no_chain():
    """R=3, L=2 (E=6), S=4, K=1 -> C=4.  Loads T = [7,3,1,0,1,0]:
    W = [10,1,1]; keep = [4,1,1]; X = [6,0,0]; D = [0,3,3].
    Donor 0 gives 3 to rank 1 then 3 to rank 2 (receivers tie on D, lower
    rank first).  Line of group 0 by (T,e): expert 1 [0,3), expert 0 [3,10);
    pieces [0,4)->0, [4,7)->1, [7,10)->2.  So rank 0 holds expert 1 (3) and
    one token of expert 0; ranks 1 and 2 hold 3 tokens of expert 0 each in
    prefetch row E+0 = 6.  With token_padding 1 the cu_seqlens follow."""
    counts = [[2, 1, 1, 0, 0, 0], [3, 1, 0, 0, 0, 0], [2, 1, 0, 0, 1, 0]]
    topk = topk_from_counts(counts, S=4, K=1)
    p = oracle.plan(topk, E=6, B=2, token_padding=1)
    check_plan(p, topk)
    assert list(p.T) == [7, 3, 1, 0, 1, 0]
    assert p.donations == [(0, 1, 3), (0, 2, 3)]
    assert list(p.keep) == [4, 1, 1]
    assert list(p.line_start[:2]) == [3, 0]
    assert p.pieces[0] == [(0, 4, 0), (4, 7, 1), (7, 10, 2)]
    assert p.cu_seqlens.tolist() == [[1, 4, 4, 4, 4, 4, 4, 4],
                                     [0, 0, 1, 1, 1, 1, 4, 4],
                                     [0, 0, 0, 0, 1, 1, 4, 4]]
    assert p.prefetch_src.tolist() == [[-1, -1], [0, -1], [0, -1]]
    assert p.dup_count == 2
    # expert 0's tokens in (r,s) order: rank0 s0,s1; rank1 s0,s1,s2; rank2 s0,s1
    # positions 3..9 -> rank 0 gets the first, rank 1 the next three, rank 2 the rest
    NvS = p.NvS
    e0 = [(r, s) for r in range(3) for s in range(4) if topk[r, s, 0] == 0]
    want = [0 * NvS + 0, 1 * NvS + 1, 1 * NvS + 2, 1 * NvS + 3,
            2 * NvS + 1, 2 * NvS + 2, 2 * NvS + 3]
    assert [p.dest[r, s, 0] for r, s in e0] == want


def test_hand_plan_with_chain():
    """R=3, L=1 (E=3), S=4, K=1 -> C=4.  T = [6,5,1]: keep = [4,4,1],
    X = [2,1,0], D = [0,0,3].  Donor 0 (x=2) meets rank 2 needing 3: it gives
    all 3, shrinks its keep to 3 and queues itself needing 1; donor 1 gives
    that 1.  Rank 0 ends with 3 of expert 0 + 1 of expert 1, rank 2 with 1 of
    expert 2 + 3 of expert 0.  Brute force agrees that 2 duplicates is the
    minimum."""
    counts = [[3, 1, 0], [2, 2, 0], [1, 2, 1]]
    topk = topk_from_counts(counts, S=4, K=1)
    p = oracle.plan(topk, E=3, B=1, token_padding=1)
    check_plan(p, topk)
    assert p.donations == [(0, 2, 3), (1, 0, 1)]
    assert list(p.keep) == [3, 4, 1]
    assert p.pieces[0] == [(0, 3, 0), (3, 6, 2)]
    assert p.pieces[1] == [(0, 4, 1), (4, 5, 0)]
    assert p.prefetch_src.tolist() == [[1], [-1], [0]]
    assert p.cu_seqlens.tolist() == [[3, 3, 3, 4], [0, 4, 4, 4], [0, 0, 1, 4]]
    assert p.dup_count == 2
    assert oracle.min_duplicates(p.T, 3, 4) == 2


def test_hand_plan_receiver_order():
    """R=3, L=1, S=4, K=1 -> C=4.  T = [8,1,3]: keep = [4,1,3], X = [4,0,0],
    D = [0,3,1].  Receivers by larger deficit first: rank 1 (3) then rank 2
    (1); pieces of expert 0's line: [0,4)->0, [4,7)->1, [7,8)->2."""
    counts = [[4, 0, 0], [3, 1, 0], [1, 0, 3]]
    topk = topk_from_counts(counts, S=4, K=1)
    p = oracle.plan(topk, E=3, B=1, token_padding=1)
    check_plan(p, topk)
    assert p.donations == [(0, 1, 3), (0, 2, 1)]
    assert p.pieces[0] == [(0, 4, 0), (4, 7, 1), (7, 8, 2)]
    assert p.cu_seqlens.tolist() == [[4, 4, 4, 4], [0, 1, 1, 4], [0, 0, 3, 4]]
    N = p.NvS
    assert p.dest[:, :, 0].tolist() == [[0, 1, 2, 3],
                                        [N + 1, N + 2, N + 3, N + 0],
                                        [2 * N + 3, 2 * N + 0, 2 * N + 1, 2 * N + 2]]


def test_hand_plan_donor_order_and_chain():
    """R=4, L=1, S=4, K=1 -> C=4.  T = [7,5,2,2]: keep = [4,4,2,2],
    X = [3,1,0,0], D = [0,0,2,2].  Donors by larger excess first: 0 (3) then
    1 (1).  Donor 0 gives 2 to rank 2 (x: 3 -> 1), then meets rank 3 needing 2
    with x = 1: it gives 2, keeps 3 and queues itself for 1, which donor 1
    supplies."""
    counts = [[4, 0, 0, 0], [3, 1, 0, 0], [0, 4, 0, 0], [0, 0, 2, 2]]
    topk = topk_from_counts(counts, S=4, K=1)
    p = oracle.plan(topk, E=4, B=1, token_padding=1)
    check_plan(p, topk)
    assert p.donations == [(0, 2, 2), (0, 3, 2), (1, 0, 1)]
    assert list(p.keep) == [3, 4, 2, 2]
    assert p.pieces[0] == [(0, 3, 0), (3, 5, 2), (5, 7, 3)]
    assert p.pieces[1] == [(0, 4, 1), (4, 5, 0)]
    assert p.prefetch_src.tolist() == [[1], [-1], [0], [0]]


def test_hand_plan_chained_rank_waits_its_turn():
    """R=4, L=1, S=4, K=1 -> C=4.  T = [6,6,1,3]: X = [2,2,0,0],
    D = [0,0,3,1].  Donor 0 (x=2) meets rank 2 needing 3: chain, rank 0 now
    needs 1 and joins the BACK of the queue, behind rank 3.  Donor 1 then
    serves rank 3 first and rank 0 second."""
    counts = [[4, 0, 0, 0], [2, 2, 0, 0], [0, 4, 0, 0], [0, 0, 1, 3]]
    topk = topk_from_counts(counts, S=4, K=1)
    p = oracle.plan(topk, E=4, B=1, token_padding=1)
    check_plan(p, topk)
    assert p.donations == [(0, 2, 3), (1, 3, 1), (1, 0, 1)]
    assert p.pieces[1] == [(0, 4, 1), (4, 5, 3), (5, 6, 0)]


def test_hand_plan_exhausted_donor_hands_over():
    """R=4, L=1, S=4, K=1 -> C=4.  T = [6,6,2,2]: X = [2,2,0,0],
    D = [0,0,2,2].  Donor 0 is used up exactly by rank 2, so donor 1 serves
    rank 3; no chain, two duplicates."""
    counts = [[4, 0, 0, 0], [2, 2, 0, 0], [0, 4, 0, 0], [0, 0, 2, 2]]
    topk = topk_from_counts(counts, S=4, K=1)
    p = oracle.plan(topk, E=4, B=1, token_padding=1)
    check_plan(p, topk)
    assert p.donations == [(0, 2, 2), (1, 3, 2)]
    assert list(p.keep) == [4, 4, 2, 2]
    assert p.dup_count == 2


# ---------------------------------------------------------- closed forms
@pytest.mark.parametrize("name", ["tiny_r4_s64_k2_e8", "mid_r8_s1024_k4_e32",
                                  "fwd_r8_s4096_k8_e256"])
def test_balanced_closed_form(name):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing_balanced(w)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    L = w.E // w.R
    tbar = w.R * w.S * w.K // w.E
    assert p.dup_count == 0 and p.donations == []
    assert (p.prefetch_src == -1).all()
    seg = round_up(tbar, w.token_padding)
    for d in range(w.R):
        for e in range(d * L, (d + 1) * L):
            assert p.cu_seqlens[d, e] == (e - d * L + 1) * seg
        assert (p.cu_seqlens[d, w.E:] == L * seg).all()
    if name != "fwd_r8_s4096_k8_e256":
        check_plan(p, topk)


def test_adversarial_closed_form_headline():
    """All tokens on experts 0..7 (group 0): W_0 = 8C.  Rank 0 keeps expert 0
    whole; donor 0 hands C to ranks 1..7 in rank order, so rank d >= 1 holds
    expert d in prefetch row E+0.  Seven duplicates, the minimum: each of the
    seven empty ranks needs at least one."""
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    topk, _ = synth.routing_adversarial(w)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    C = w.S * w.K
    assert p.dup_count == w.R - 1
    assert p.cu_seqlens[0, 0] == C and (p.cu_seqlens[0] == C).all()
    for d in range(1, w.R):
        assert p.prefetch_src[d, 0] == d and (p.prefetch_src[d, 1:] == -1).all()
        assert (p.cu_seqlens[d, : w.E] == 0).all()
        assert (p.cu_seqlens[d, w.E:] == C).all()
    # and it is a valid plan (checked on the counts-level structure only,
    # the full per-token check is O(R*S*K*E) here)
    assert ((p.src >= 0).sum(axis=1) == C).all()


def test_nvs_values():
    got = {n: oracle.nvs(w.S, w.K, w.E, w.R, w.token_padding)
           for n, w in synth.WORKLOADS.items()}
    assert got["tiny_r4_s64_k2_e8"] == 192
    assert got["mid_r8_s1024_k4_e32"] == 5120
    assert got["fwd_r8_s4096_k8_e256"] == 40960
    assert got["infer_r8_s128_k8_e256_b4"] == 9216


# ---------------------------------------------------------- invariants
@pytest.mark.parametrize("name,target", [
    (n, t) for n, ts in synth.SWEEPS.items() for t in ts
    if not n.startswith("fwd_")])
def test_invariants_on_workloads(name, target):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    check_plan(p, topk)
    if w.B == w.E // w.R:
        assert all(len(x) <= w.B for x in p.remote_experts)


def random_instance(rng):
    R = int(rng.integers(1, 7))
    L = int(rng.integers(1, 5))
    E = R * L
    K = int(rng.integers(1, min(E, 4) + 1))
    S = int(rng.integers(1, 40))
    skew = float(rng.uniform(0, 3))
    logits = rng.standard_normal((R, S, E)) - skew * np.log1p(np.arange(E))
    if rng.random() < 0.3:
        logits = logits[..., rng.permutation(E)]
    topk = np.argsort(-logits, axis=-1, kind="stable")[..., :K].astype(np.int32)
    B = int(rng.integers(0, L + 1)) if rng.random() < 0.3 else L
    tp = int(rng.choice([1, 2, 3, 8]))
    return topk, E, B, tp


def test_invariants_random_instances():
    rng = np.random.default_rng(2024)
    for _ in range(300):
        topk, E, B, tp = random_instance(rng)
        p = oracle.plan(topk, E, B, tp)
        check_plan(p, topk)


def test_one_rank_is_identity_layout():
    rng = np.random.default_rng(5)
    topk = np.argsort(-rng.standard_normal((1, 10, 4)), axis=-1)[..., :2].astype(np.int32)
    p = oracle.plan(topk, E=4, B=4, token_padding=1)
    check_plan(p, topk)
    assert p.dup_count == 0 and p.donations == []


def test_bad_routing_rejected():
    with pytest.raises(ValueError):
        oracle.plan(np.array([[[0, 0]]], dtype=np.int32), E=2, B=1, token_padding=1)
    with pytest.raises(ValueError):
        oracle.plan(np.array([[[0, 5]]], dtype=np.int32), E=2, B=1, token_padding=1)


# ---------------------------------------------------------- brute force
@pytest.mark.parametrize("R,L,S,K,n", [(3, 2, 6, 2, 40), (4, 2, 8, 2, 25), (3, 1, 5, 1, 40)])
def test_near_optimal_against_brute_force(R, L, S, K, n):
    """The planner never beats the exact optimum (sanity of both) and is at
    most R-1 redundant experts above it (the reading of 'near-optimal')."""
    rng = np.random.default_rng(R * 100 + L * 10 + S)
    E = R * L
    gaps = []
    for i in range(n):
        s = float(rng.uniform(0, 2.5))
        logits = rng.standard_normal((R, S, E)) - s * np.log1p(np.arange(E))
        logits = logits[..., rng.permutation(E)]
        topk = np.argsort(-logits, axis=-1, kind="stable")[..., :K].astype(np.int32)
        p = oracle.plan(topk, E, L, 1)
        opt = oracle.min_duplicates(p.T, R, S * K)
        assert opt <= p.dup_count <= opt + R - 1
        gaps.append(p.dup_count - opt)
    assert min(gaps) == 0


def test_brute_force_closed_forms():
    # balanced: nothing to move
    assert oracle.min_duplicates([2, 2, 2, 2], R=2, C=4) == 0
    # group 0 holds everything: each of the other ranks needs >= 1 duplicate
    assert oracle.min_duplicates([6, 6, 0, 0, 0, 0], R=3, C=4) == 2
    # a single hot expert spread over two other ranks plus its home
    assert oracle.min_duplicates([9, 0, 0, 0, 3, 0], R=3, C=4) == 2
