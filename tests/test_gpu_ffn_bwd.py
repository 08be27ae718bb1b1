"""Backward of the grouped SwiGLU FFN on the GPU (moonep_expert_ffn_bwd)
against the oracle (oracle.expert_ffn_backward: float64 products, dZ, dG, dU
and dX rounded to bf16 where stored).

Tolerance: rel-L2 <= 1e-2 per output; element-wise <= max(2e-2, 1 bf16 ulp)
for dZ (one product, as the forward) and max(2e-2, 2 ulps) for dG, dU and dX,
which are computed from the rounded dZ (resp. dG, dU) of each side.
Also: slots outside segments untouched, dX in place over dY, single-rank
calls, and the full-size configuration on sampled rows.
"""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import assert_close_bf16, buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu

SENT = 0x7F7F


def _sentinel(shape):
    return torch.full(shape, SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _inputs(w, target, seed=5):
    if isinstance(target, tuple):                 # ("zipf", s): Zipf strength s, seed 7
        topk, _ = synth.routing_zipf(w, target[1], seed=7)
    else:
        topk, _ = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs, _ = oracle.dispatch(p, synth.hidden(w))
    rng = np.random.default_rng(seed)
    dy = oracle.f32_to_bf16(rng.standard_normal((w.R, p.NvS, w.H)).astype(np.float32))
    dy[p.src < 0] = 0
    home_h = [synth.expert_weights_host(w, i) for i in range(3)]
    pool_h = [oracle.prefetch_weight(p, home_h[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
              for i in range(3)]
    return topk, p, x_nvs, dy, home_h, pool_h


@pytest.mark.parametrize("name,target,ranks", [
    ("tiny_r4_s64_k2_e8", 1.0, None), ("tiny_r4_s64_k2_e8", 0.0, None),
    ("tiny_r4_s64_k2_e8", "adv", None),
    ("mid_r8_s1024_k4_e32", 0.0, [0, 6]), ("mid_r8_s1024_k4_e32", 2.0, [1, 4]),
    ("mid_r8_s1024_k4_e32", ("zipf", 2.0), [3, 6]),   # segments of 9-16 full tiles
])
def test_ffn_bwd_matches_oracle(name, target, ranks):
    w = synth.WORKLOADS[name]
    log(f"ffn bwd {name} target={target}")
    topk, p, x_nvs, dy, home_h, pool_h = _inputs(w, target)
    want = oracle.expert_ffn_backward(p, x_nvs, dy, home_h, pool_h, ranks=ranks)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    buf.prefetch_weight(plan, home, pool)
    outs = [_sentinel((w.R, buf.NvS, W)) for W in (w.Hp, w.Hp, w.Hp, w.H)]
    buf.expert_ffn_bwd(plan, dev_bf16(x_nvs), dev_bf16(dy), home, pool, *outs)
    got = [host_bf16(o) for o in outs]
    names = ("dz", "dg", "du", "dx")
    for d in (range(w.R) if ranks is None else ranks):
        end = p.cu_seqlens[d, -1]
        for nm, g_, w_ in zip(names, got, want):
            assert_close_bf16(g_[d, :end], w_[d, :end], what=f"{nm} rank {d}",
                              ulps=1 if nm == "dz" else 2)
            assert (g_[d, end:] == SENT).all(), f"{nm} rank {d} written past the last segment"
        pad = p.src[d, :end] < 0
        assert (got[3][d, :end][pad] == 0).all()
    buf.destroy()


def test_ffn_bwd_in_place_and_single_rank():
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    topk, p, x_nvs, dy, home_h, pool_h = _inputs(w, 1.0, seed=6)
    _, _, _, dx_want = oracle.expert_ffn_backward(p, x_nvs, dy, home_h, pool_h)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    buf.prefetch_weight(plan, home, pool)
    dy_d = dev_bf16(dy)
    for d in range(w.R):
        buf.expert_ffn_bwd(plan, dev_bf16(x_nvs), dy_d, home, pool, dx_nvs=dy_d, rank=d)
    got = host_bf16(dy_d)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert_close_bf16(got[d, :end], dx_want[d, :end], what=f"in-place dx rank {d}", ulps=2)
    buf.destroy()


def test_ffn_bwd_rejects_aliased_workspaces():
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    topk, p, x_nvs, dy, home_h, pool_h = _inputs(w, 1.0)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    ws = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device="cuda")
    from grouped_gemm_moonep_amd import MoonepError
    with pytest.raises(MoonepError):
        buf.expert_ffn_bwd(plan, dev_bf16(x_nvs), dev_bf16(dy), home, pool, dz_ws=ws, dg_nvs=ws)
    buf.destroy()


@pytest.mark.parametrize("target", [0.0, 2.0, "adv"])
def test_ffn_bwd_full_size_sampled(target):
    """Headline shapes: weights drawn on the GPU; the oracle recomputes sampled
    rows of sampled segments from the home weights (the backward is row-wise).
    Balanced, Zipf (maxvio 2) and adversarial routing (one 32768-row segment
    per rank)."""
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    log(f"ffn bwd full size target={target}")
    topk, _ = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    for i in range(3):
        synth.expert_weights_device(w, i, home[i])
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((w.R, w.S, w.H), generator=g, device="cuda").to(torch.bfloat16)
    dout = torch.randn((w.R, w.S, w.H), generator=g, device="cuda").to(torch.bfloat16)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, x)
    dy_nvs, _ = buf.dispatch(plan, dout)
    buf.prefetch_weight(plan, home, pool)
    dz, dg, du, dx = buf.expert_ffn_bwd(plan, x_nvs, dy_nvs, home, pool)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    segs = [(d, row) for d in range(w.R) for row in range(w.E + w.B) if p.seg_tokens[d, row] > 0]
    pick = [segs[i] for i in rng.choice(len(segs), min(5, len(segs)), replace=False)]
    xs = host_bf16(x).reshape(-1, w.H)
    ds = host_bf16(dout).reshape(-1, w.H)
    for d, row in pick:
        e = row if row < w.E else p.prefetch_src[d, row - w.E]
        end = p.cu_seqlens[d, row]
        start = end - p.seg_len[d, row]
        n_pick = min(48 if p.seg_tokens[d, row] > 4096 else 16, p.seg_tokens[d, row])
        slots = start + rng.choice(p.seg_tokens[d, row], n_pick, replace=False)
        toks = p.src[d, slots] // w.K
        wts = [host_bf16(home[i][e]) for i in range(3)]
        want = oracle.ffn_token_backward(xs[toks], ds[toks], *wts)
        for nm, t, ref in zip(("dz", "dg", "du", "dx"), (dz, dg, du, dx), want):
            assert_close_bf16(host_bf16(t[d, slots]), ref, what=f"{nm} d={d} row={row}",
                              ulps=1 if nm == "dz" else 2)
    buf.destroy()


@pytest.mark.parametrize("name,target", [("tiny_r4_s64_k2_e8", 1.0), ("bwd_r8_s1024_k4_e32", 2.0)])
def test_training_step_equals_dense(name, target):
    """A whole training step of the MoE layer with an unweighted combine
    (out = sum_k FFN_k(x)): forward, combine bwd (dispatch of dOut), FFN
    backward, dispatch bwd (unweighted combine), weight gradients and
    reduce_grad -- against a dense per-token computation that never sees a
    plan: dx = sum_k dX_k (fp32, ascending k, bf16), dW_e = sum over the
    tokens routed to e of the per-token weight gradients."""
    w = synth.WORKLOADS[name]
    log(f"training step {name} target={target}")
    topk, _ = synth.routing(w, target)
    x = synth.hidden(w)
    dout = synth.grad_out(w, w.H)
    home_h = [synth.expert_weights_host(w, i) for i in range(3)]
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    home = [dev_bf16(h) for h in home_h]
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    buf.prefetch_weight(plan, home, pool)
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x))
    z, y = buf.expert_ffn(plan, x_nvs, home, pool)
    dy_nvs, _ = buf.dispatch(plan, dev_bf16(dout))                    # combine bwd
    _, dg, du, dx_nvs = buf.expert_ffn_bwd(plan, x_nvs, dy_nvs, home, pool)
    dx, _ = buf.combine(plan, dx_nvs)                                 # dispatch bwd
    grads = [torch.zeros((w.E, w.H, w.Hp), dtype=torch.float32, device="cuda") for _ in range(3)]
    rbuf = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.float32, device="cuda")
            for _ in range(3)]
    buf.expert_wgrad(plan, x_nvs, dg, grads[0], rbuf[0])
    buf.expert_wgrad(plan, x_nvs, du, grads[1], rbuf[1])
    buf.expert_wgrad(plan, dy_nvs, z, grads[2], rbuf[2])
    buf.reduce_grad(plan, grads, rbuf)
    torch.cuda.synchronize()

    # dense reference, token-major
    R, S, K, E = w.R, w.S, w.K, w.E
    xt = x.reshape(R * S, w.H)
    dt = dout.reshape(R * S, w.H)
    ids = topk.reshape(R * S, K)
    dx_k = np.zeros((R * S, K, w.H), dtype=np.uint16)
    f = lambda b: oracle.bf16_to_f32(b).astype(np.float64)
    gw = [np.zeros((E, w.H, w.Hp)) for _ in range(3)]
    for e in range(E):
        t, k = np.nonzero(ids == e)
        if t.size == 0:
            continue
        dz_e, dg_e, du_e, dx_e = oracle.ffn_token_backward(xt[t], dt[t], home_h[0][e],
                                                           home_h[1][e], home_h[2][e])
        z_e, _ = oracle.ffn_token(xt[t], home_h[0][e], home_h[1][e], home_h[2][e])
        dx_k[t, k] = dx_e
        gw[0][e] = f(xt[t]).T @ f(dg_e)
        gw[1][e] = f(xt[t]).T @ f(du_e)
        gw[2][e] = f(dt[t]).T @ f(z_e)
    dx_want = oracle.combine_rows(dx_k).reshape(R, S, w.H)
    assert_close_bf16(host_bf16(dx), dx_want, what="dx", ulps=2)
    for i, nm in enumerate(("dWg", "dWu", "dWd")):
        got = grads[i].cpu().numpy().astype(np.float64)
        scale = max(np.abs(gw[i]).max(), 1.0)
        err = np.abs(got - gw[i]).max() / scale
        rel = np.linalg.norm(got - gw[i]) / max(np.linalg.norm(gw[i]), 1e-30)
        assert rel <= 1e-2 and err <= 2e-2, f"{nm}: rel-L2 {rel:.2e}, max-abs/scale {err:.2e}"
    buf.destroy()
