"""moonep_plan on the GPU against the oracle planner, bit for bit: counts,
dest, src, cu_seqlens, seg_tokens, prefetch_src and the stats, at every
workload and imbalance point, plus edge shapes and bad routing."""
import dataclasses

import numpy as np
import pytest

import moonep_synth as synth
import oracle
from gpu_util import buffer_for, dev, log, plan_host
from plan_checks import check_plan_arrays

pytestmark = pytest.mark.gpu


def run_and_compare(w, topk, tpe=None, full_check=True):
    log(f"plan {w.name} R={w.R} S={w.S} K={w.K} E={w.E} B={w.B} tp={w.token_padding}")
    buf = buffer_for(w)
    plan = buf.plan(dev(topk), None if tpe is None else dev(tpe))
    got = plan_host(buf, plan)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    assert got["stats"][0] == 0
    for name in ("counts", "cu_seqlens", "seg_tokens", "prefetch_src", "dest", "src"):
        want = getattr(p, name)
        assert np.array_equal(got[name], want), name
    st = got["stats"]
    assert st[1] == p.dup_count
    assert st[2] == p.T.max()
    assert st[3] == len(p.donations)
    assert st[4] == int((p.seg_len - p.seg_tokens).sum())
    mv = np.frombuffer(np.int32(st[5]).tobytes(), np.float32)[0]
    assert abs(mv - oracle.maxvio(topk, w.E)) <= 1e-5 * max(1.0, abs(mv))
    assert list(st[8:8 + w.R]) == [int(g) for g in p.remote_group]
    assert list(st[8 + w.R:8 + 2 * w.R]) == [len(x) for x in p.remote_experts]
    if full_check:
        check_plan_arrays(topk, w.E, w.B, w.token_padding, p.NvS, got["dest"], got["src"],
                          got["cu_seqlens"], got["seg_tokens"], got["prefetch_src"])
    buf.destroy()
    return got


FULL = ("fwd_", "pages_")


@pytest.mark.parametrize("name,target", [
    (n, t) for n, ts in synth.SWEEPS.items() for t in ts if not n.startswith(FULL)])
def test_plan_matches_oracle(name, target):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing(w, target)
    run_and_compare(w, topk)


@pytest.mark.parametrize("name,target", [
    (n, t) for n, ts in synth.SWEEPS.items() for t in ts if n.startswith(FULL)])
def test_plan_matches_oracle_full_size(name, target):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing(w, target)
    run_and_compare(w, topk, full_check=False)


def test_plan_with_tokens_per_expert():
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    topk, _ = synth.routing(w, 1.0)
    counts = np.stack([np.bincount(topk[r].reshape(-1), minlength=w.E) for r in range(w.R)])
    run_and_compare(w, topk, tpe=counts.astype(np.int32))


EDGE = [
    synth.Workload("r1", R=1, S=100, K=3, E=8, B=8, H=64, Hp=64, token_padding=4),
    synth.Workload("k1", R=4, S=300, K=1, E=8, B=2, H=64, Hp=64, token_padding=8),
    synth.Workload("k_eq_e", R=2, S=70, K=6, E=6, B=3, H=64, Hp=64, token_padding=1),
    synth.Workload("tp1", R=8, S=513, K=4, E=64, B=8, H=64, Hp=64, token_padding=1),
    synth.Workload("b0", R=4, S=257, K=2, E=16, B=0, H=64, Hp=64, token_padding=16),
    synth.Workload("s1", R=3, S=1, K=2, E=6, B=2, H=64, Hp=64, token_padding=2),
    synth.Workload("l1", R=16, S=200, K=4, E=16, B=1, H=64, Hp=64, token_padding=8),
    synth.Workload("wide", R=8, S=600, K=8, E=1024, B=128, H=64, Hp=64, token_padding=32),
    synth.Workload("r64", R=64, S=40, K=2, E=128, B=2, H=64, Hp=64, token_padding=4),
    synth.Workload("tp384", R=4, S=200, K=3, E=8, B=2, H=64, Hp=64, token_padding=384),
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
@pytest.mark.parametrize("s", [0.0, 1.5])
def test_plan_edge_shapes(w, s):
    topk, _ = synth.routing_zipf(w, s, seed=7)
    run_and_compare(w, topk)


def test_plan_long_sequence():
    """S = 32768 tokens per rank: 128 planning chunks per rank, so the chunk
    sums and the assignment's chunk bases take several rounds of loads."""
    w = synth.Workload("long_r8_s32768_k8_e256", R=8, S=32768, K=8, E=256, B=32, H=64, Hp=64,
                       token_padding=128)
    topk, _ = synth.routing_zipf(w, 0.4, seed=3)
    run_and_compare(w, topk, full_check=False)


def test_plan_adversarial_small():
    w = dataclasses.replace(synth.WORKLOADS["mid_r8_s1024_k4_e32"], name="adv")
    topk, _ = synth.routing_adversarial(w)
    run_and_compare(w, topk)


@pytest.mark.parametrize("kind", ["range", "repeat", "counts"])
def test_bad_routing_sets_flag_and_safe_plan(kind):
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    topk, _ = synth.routing(w, 1.0)
    topk = topk.copy()
    tpe = None
    if kind == "range":
        topk[1, 5, 0] = w.E + 3
        bit = 1
    elif kind == "repeat":
        topk[2, 7, 1] = topk[2, 7, 0]
        bit = 2
    else:
        tpe = np.zeros((w.R, w.E), np.int32)
        bit = 4
    log(f"bad routing {kind}")
    buf = buffer_for(w)
    plan = buf.plan(dev(topk), None if tpe is None else dev(tpe))
    got = plan_host(buf, plan)
    assert got["stats"][0] & bit
    assert (got["cu_seqlens"] == 0).all() and (got["prefetch_src"] == -1).all()
    assert (got["src"] == -1).all()
    R, S, K = topk.shape
    NvS = buf.NvS
    want = (np.arange(R)[:, None, None] * NvS + np.arange(S * K).reshape(S, K)[None])
    assert np.array_equal(got["dest"], want)
    buf.destroy()
