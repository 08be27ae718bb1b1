"""The grouped SwiGLU FFN and the whole forward path on the GPU.

* moonep_expert_ffn against the oracle's grouped FFN (float64 products, bf16
  Z and Y) on every segment: rel-L2 <= 1e-2 and max-abs <= 2e-2;
* slots outside segments are not written; y may alias x (in place);
* plan -> dispatch -> prefetch -> FFN -> combine against the dense,
  unbalanced per-token MoE (no planner involved) at the same tolerance;
* the full-size forward config checked on sampled rows of sampled segments
  (balanced, Zipf and adversarial routing) and end to end on sampled tokens
  against the dense MoE.
"""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import assert_close_bf16, buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu

SENT = 0x7F7F


def _setup(w, target):
    # a float target is a maxvio of the workload's sweep; ("zipf", s) draws
    # Zipf-biased routing of strength s directly (seed 7)
    if isinstance(target, tuple):
        topk, rw = synth.routing_zipf(w, target[1], seed=7)
    else:
        topk, rw = synth.routing(w, target)
    x = synth.hidden(w)
    home_h = [synth.expert_weights_host(w, i) for i in range(3)]
    return topk, rw, x, home_h


def _pool_dev(w):
    return [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]


@pytest.mark.parametrize("name,target,ranks", [
    ("tiny_r4_s64_k2_e8", 1.0, None), ("tiny_r4_s64_k2_e8", 0.0, None),
    ("tiny_r4_s64_k2_e8", "adv", None),
    ("mid_r8_s1024_k4_e32", 0.0, [0, 5]), ("mid_r8_s1024_k4_e32", 2.0, [0, 3, 7]),
    # maxvio 7: segments of 9 to 16 full tiles, split into uneven groups of up
    # to 8 (rank 3: 15 and a short tail, rank 5: 16, rank 6: 9 and a tail)
    ("mid_r8_s1024_k4_e32", ("zipf", 2.0), [3, 5, 6]),
])
def test_ffn_matches_oracle(name, target, ranks):
    w = synth.WORKLOADS[name]
    log(f"ffn {name} target={target}")
    topk, rw, x, home_h = _setup(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs_h, _ = oracle.dispatch(p, x)
    pool_h = [oracle.prefetch_weight(p, home_h[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
              for i in range(3)]
    z_want, y_want = oracle.expert_ffn(p, x_nvs_h, home_h, pool_h, ranks=ranks)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = _pool_dev(w)
    buf.prefetch_weight(plan, home, pool)
    x_nvs = dev_bf16(x_nvs_h)
    z = torch.full((w.R, buf.NvS, w.Hp), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    y = torch.full((w.R, buf.NvS, w.H), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    buf.expert_ffn(plan, x_nvs, home, pool, z, y)
    zg, yg = host_bf16(z), host_bf16(y)
    for d in (range(w.R) if ranks is None else ranks):
        end = p.cu_seqlens[d, -1]
        assert_close_bf16(zg[d, :end], z_want[d, :end], what=f"z rank {d}")
        assert_close_bf16(yg[d, :end], y_want[d, :end], what=f"y rank {d}")
        assert (yg[d, end:] == SENT).all() and (zg[d, end:] == SENT).all()
        pad = p.src[d, :end] < 0
        assert (yg[d, :end][pad] == 0).all()
    buf.destroy()


def test_ffn_single_rank_and_in_place():
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    topk, rw, x, home_h = _setup(w, "adv")
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs_h, _ = oracle.dispatch(p, x)
    pool_h = [oracle.prefetch_weight(p, home_h[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
              for i in range(3)]
    _, y_want = oracle.expert_ffn(p, x_nvs_h, home_h, pool_h)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = _pool_dev(w)
    buf.prefetch_weight(plan, home, pool)
    x_nvs = dev_bf16(x_nvs_h)
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device="cuda")
    for d in range(w.R):
        buf.expert_ffn(plan, x_nvs, home, pool, z, x_nvs, rank=d)   # y aliases x
    yg = host_bf16(x_nvs)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert_close_bf16(yg[d, :end], y_want[d, :end], what=f"in-place rank {d}")
    buf.destroy()


@pytest.mark.parametrize("name,target", [
    ("tiny_r4_s64_k2_e8", 1.0), ("tiny_r4_s64_k2_e8", 0.0), ("tiny_r4_s64_k2_e8", "adv"),
    ("mid_r8_s1024_k4_e32", 1.0),
])
def test_forward_equals_dense_moe(name, target):
    w = synth.WORKLOADS[name]
    log(f"forward {name} target={target}")
    topk, rw, x, home_h = _setup(w, target)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = _pool_dev(w)
    x_nvs, rw_nvs = buf.dispatch(plan, dev_bf16(x), dev(rw))
    buf.prefetch_weight(plan, home, pool)
    z, y = buf.expert_ffn(plan, x_nvs, home, pool, y_nvs=x_nvs)
    out, rw_sk = buf.combine(plan, y, rw_nvs)
    got = host_bf16(out)
    if name.startswith("mid"):
        rows = np.random.default_rng(0).choice(w.R * w.S, 256, replace=False)
        r_, s_ = rows // w.S, rows % w.S
        want = oracle.dense_moe(topk[r_, s_][None], rw[r_, s_][None], x[r_, s_][None], home_h)[0]
        assert_close_bf16(got[r_, s_], want, what="forward sampled")
    else:
        want = oracle.dense_moe(topk, rw, x, home_h)
        assert_close_bf16(got, want, what="forward")
    assert np.array_equal(rw_sk.cpu().numpy(), rw)
    buf.destroy()


def test_inference_overflow_forward():
    """B < E/R: overflow experts read their home rows through cu_seqlens."""
    w = synth.Workload("infer_small", R=4, S=64, K=4, E=32, B=1, H=128, Hp=128,
                       token_padding=16)
    topk, rw = synth.routing_zipf(w, 1.5)
    x = synth.hidden(w)
    home_h = [synth.expert_weights_host(w, i) for i in range(3)]
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    assert max(len(r) for r in p.remote_experts) > w.B
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = _pool_dev(w)
    x_nvs, rw_nvs = buf.dispatch(plan, dev_bf16(x), dev(rw))
    buf.prefetch_weight(plan, home, pool)
    _, y = buf.expert_ffn(plan, x_nvs, home, pool)
    out, _ = buf.combine(plan, y, rw_nvs)
    assert_close_bf16(host_bf16(out), oracle.dense_moe(topk, rw, x, home_h), what="overflow")
    buf.destroy()


@pytest.mark.parametrize("name,target", [("fwd_r8_s4096_k8_e256", 0.0),
                                         ("fwd_r8_s4096_k8_e256", 2.0),
                                         ("fwd_r8_s4096_k8_e256", "adv"),
                                         ("infer_r8_s128_k8_e256_b4", 4.0),
                                         ("pages_r8_s8192_k8_e384", 10.0)])
def test_ffn_full_size_sampled(name, target):
    """Full-size weights drawn on the GPU; the oracle recomputes sampled rows
    of sampled segments token by token from the home weights.  At the
    headline: balanced routing (whole 256-row tiles, no padding), Zipf
    routing at maxvio 2, and the adversarial case, where each rank holds one
    32768-row segment that the tile schedule splits into 16 groups of 8
    tiles (rows sampled across the whole segment)."""
    w = synth.WORKLOADS[name]
    log(f"ffn full size {name} target={target}")
    topk, rw = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    for i in range(3):
        synth.expert_weights_device(w, i, home[i])
    pool = _pool_dev(w)
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((w.R, w.S, w.H), generator=g, device="cuda").to(torch.bfloat16)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, x)
    buf.prefetch_weight(plan, home, pool)
    z, y = buf.expert_ffn(plan, x_nvs, home, pool)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    segs = [(d, row) for d in range(w.R) for row in range(w.E + w.B) if p.seg_tokens[d, row] > 0]
    pick = [segs[i] for i in rng.choice(len(segs), min(6, len(segs)), replace=False)]
    xs = host_bf16(x).reshape(-1, w.H)
    for d, row in pick:
        e = row if row < w.E else p.prefetch_src[d, row - w.E]
        end = p.cu_seqlens[d, row]
        start = end - p.seg_len[d, row]
        n_pick = min(64 if p.seg_tokens[d, row] > 4096 else 16, p.seg_tokens[d, row])
        slots = start + rng.choice(p.seg_tokens[d, row], n_pick, replace=False)
        toks = p.src[d, slots] // w.K
        wts = [host_bf16(home[i][e]) for i in range(3)]
        zw, yw = oracle.ffn_token(xs[toks], *wts)
        assert_close_bf16(host_bf16(z[d, slots]), zw, what=f"z d={d} row={row}")
        assert_close_bf16(host_bf16(y[d, slots]), yw, what=f"y d={d} row={row}")
    buf.destroy()


class _DeviceRows:
    """home[e] of a device weight tensor, copied to the host on first use (the
    dense reference needs only the experts of the sampled tokens)."""

    def __init__(self, t):
        self.t, self.cache = t, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = host_bf16(self.t[e])
        return self.cache[e]


@pytest.mark.parametrize("target,ntok", [("adv", 64), (0.0, 3), (2.0, 3)])
def test_forward_full_size_equals_dense_sampled(target, ntok):
    """The headline forward end to end (plan -> dispatch -> prefetch -> FFN in
    place -> weighted combine, all 8 ranks at full size) on sampled tokens
    against the dense per-token MoE, which never sees the plan; the gathered
    route weights bit-exact for every token."""
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    log(f"forward full size {w.name} target={target}")
    topk, rw = synth.routing(w, target)
    home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    for i in range(3):
        synth.expert_weights_device(w, i, home[i])
    pool = _pool_dev(w)
    g = torch.Generator(device="cuda").manual_seed(13)
    x = torch.randn((w.R, w.S, w.H), generator=g, device="cuda").to(torch.bfloat16)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, rw_nvs = buf.dispatch(plan, x, dev(rw))
    buf.prefetch_weight(plan, home, pool)
    buf.expert_ffn(plan, x_nvs, home, pool, y_nvs=x_nvs)
    out, rw_sk = buf.combine(plan, x_nvs, rw_nvs)
    torch.cuda.synchronize()
    assert np.array_equal(rw_sk.cpu().numpy(), rw)
    rows = np.random.default_rng(14).choice(w.R * w.S, ntok, replace=False)
    r_, s_ = rows // w.S, rows % w.S
    xh = host_bf16(x[torch.from_numpy(r_).cuda(), torch.from_numpy(s_).cuda()])
    want = oracle.dense_moe(topk[r_, s_][None], rw[r_, s_][None], xh[None],
                            [_DeviceRows(t) for t in home])[0]
    got = host_bf16(out[torch.from_numpy(r_).cuda(), torch.from_numpy(s_).cuda()])
    assert_close_bf16(got, want, what=f"forward full size {target}")
    buf.destroy()


def test_gateup_then_down_equals_ffn():
    """moonep_expert_gateup + moonep_expert_down are the two launches of
    moonep_expert_ffn: identical bits, and each touches only its output."""
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    topk, rw, x, home_h = _setup(w, 2.0)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = _pool_dev(w)
    buf.prefetch_weight(plan, home, pool)
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x))
    z1, y1 = buf.expert_ffn(plan, x_nvs, home, pool)
    z2 = torch.full_like(z1, 0).view(torch.int16).fill_(SENT).view(torch.bfloat16)
    buf.expert_gateup(plan, x_nvs, [home[0], home[1], None], [pool[0], pool[1], None], z2)
    y2 = torch.full_like(y1, 0).view(torch.int16).fill_(SENT).view(torch.bfloat16)
    buf.expert_down(plan, z2, [None, None, home[2]], [None, None, pool[2]], y2)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    z1h, z2h, y1h, y2h = host_bf16(z1), host_bf16(z2), host_bf16(y1), host_bf16(y2)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert np.array_equal(z1h[d, :end], z2h[d, :end])
        assert np.array_equal(y1h[d, :end], y2h[d, :end])
        assert (z2h[d, end:] == SENT).all() and (y2h[d, end:] == SENT).all()
    buf.destroy()
