"""Seeded random shapes through the whole path against the oracle: ranks 1-8,
1-4 home experts per rank, K up to 8, 0 to E/R prefetch slots, token
padding 1-128, hidden and FFN widths any multiple of 64 up to 1024; Zipf
routing strength 0-3 in the first 24 cases, then rank-skewed routing (every
rank sends to the next rank's experts), hot experts in every token and all
tokens on the first K experts.  Each case checks dispatch (bit-exact on every used
slot), the grouped FFN (rel-L2 <= 1e-2 and max(2e-2, 1 ulp)), combine of the
oracle's FFN output (bit-exact) and, where B = E/R, the FFN backward (2 ulps
for dG, dU, dX).  The shapes mix segment lengths that leave every kind of
tile: full, partial, short tails, long segments split into groups."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import assert_close_bf16, buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu


def _shape(case):
    rng = np.random.default_rng([20261203, case])
    R = int(rng.choice([1, 2, 3, 4, 8]))
    L = int(rng.choice([1, 2, 3, 4]))
    E = R * L
    K = int(rng.integers(1, min(E, 8) + 1))
    B = int(rng.integers(0, L + 1))
    S = int(rng.integers(1, 2000))
    H = 64 * int(rng.integers(1, 17))
    Hp = 64 * int(rng.integers(1, 17))
    tp = int(rng.choice([1, 2, 4, 16, 64, 128]))
    s = float(rng.choice([0.0, 0.5, 1.5, 3.0]))
    return synth.Workload(f"rand{case}", R=R, S=S, K=K, E=E, B=B, H=H, Hp=Hp, token_padding=tp), s


def _routing(w, s, case):
    if case < 24:
        return synth.routing_zipf(w, s, seed=case), f"zipf s={s}"
    kind = case % 3
    if kind == 0:
        return synth.routing_rank_skew(w, 1.0 + s, seed=case), f"rank-skew {1.0 + s}"
    if kind == 1:
        nhot = 1 + case % w.K
        return synth.routing_hot(w, nhot, seed=case), f"hot {nhot}"
    return synth.routing_adversarial(w, seed=case), "adversarial"


@pytest.mark.parametrize("case", range(36))
def test_random_shape_path(case):
    w, s = _shape(case)
    R, B, H, Hp = w.R, w.B, w.H, w.Hp
    (topk, rw), desc = _routing(w, s, case)
    log(f"random shape {case}: {w} {desc}")
    p = oracle.plan(topk, w.E, B, w.token_padding)
    x = synth.hidden(w)
    x_nvs, rw_nvs = oracle.dispatch(p, x, rw)
    home = [synth.expert_weights_host(w, i) for i in range(3)]
    pool = [oracle.prefetch_weight(p, home[i], np.zeros((R, B, H, Hp), np.uint16)) for i in range(3)]
    z_want, y_want = oracle.expert_ffn(p, x_nvs, home, pool)
    out_want, _ = oracle.combine(p, y_want, rw_nvs)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home_d = [dev_bf16(h) for h in home]
    pool_d = [torch.zeros((R, B, H, Hp), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    buf.prefetch_weight(plan, home_d, pool_d)
    xg, rwg = buf.dispatch(plan, dev_bf16(x), dev(rw))
    xgh = host_bf16(xg)
    z, y = buf.expert_ffn(plan, xg, home_d, pool_d)
    zh, yh = host_bf16(z), host_bf16(y)
    for d in range(R):
        end = p.cu_seqlens[d, -1]
        assert np.array_equal(xgh[d, :end], x_nvs[d, :end]), f"dispatch rank {d}"
        assert_close_bf16(zh[d, :end], z_want[d, :end], what=f"z rank {d}")
        assert_close_bf16(yh[d, :end], y_want[d, :end], what=f"y rank {d}")
    out, _ = buf.combine(plan, dev_bf16(y_want), rwg)
    assert np.array_equal(host_bf16(out), out_want)
    if B == w.E // R:
        dy_nvs, _ = oracle.dispatch(p, synth.grad_out(w, H))
        want = oracle.expert_ffn_backward(p, x_nvs, dy_nvs, home, pool)
        got = buf.expert_ffn_bwd(plan, dev_bf16(x_nvs), dev_bf16(dy_nvs), home_d, pool_d)
        for nm, g_, w_ in zip(("dz", "dg", "du", "dx"), got, want):
            gh = host_bf16(g_)
            for d in range(R):
                end = p.cu_seqlens[d, -1]
                assert_close_bf16(gh[d, :end], w_[d, :end], what=f"{nm} rank {d}",
                                  ulps=1 if nm == "dz" else 2)
    buf.destroy()
