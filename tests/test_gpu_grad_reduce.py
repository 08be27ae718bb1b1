"""Training backward on the GPU: combine bwd (dispatch of dY), weight
gradients into the fp32 [E+B] gradient buffer (prefetch rows in the reduce
buffer), reduce_grad into home rows, and the reduce slots zeroed.

* moonep_expert_wgrad against the oracle (float64 products): rel-L2 <= 1e-2,
  max-abs <= 2e-2 relative to the gradient scale;
* moonep_reduce_grad against the oracle's fp32 ascending-rank sum: within
  1e-6 relative, used slots exactly zero, unused slots untouched;
* after both, home rows equal the dense per-expert gradient."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import buffer_for, dev, dev_bf16, host_bf16, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,target", [
    ("tiny_r4_s64_k2_e8", 1.0), ("tiny_r4_s64_k2_e8", "adv"),
    ("bwd_r8_s1024_k4_e32", 0.0), ("bwd_r8_s1024_k4_e32", 2.0)])
def test_wgrad_and_reduce(name, target):
    w = synth.WORKLOADS[name]
    log(f"wgrad+reduce {name} target={target}")
    topk, _ = synth.routing(w, target)
    x = synth.hidden(w)
    dy = synth.grad_out(w, w.Hp)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    rng = np.random.default_rng(8)
    gh0 = rng.standard_normal((w.E, w.H, w.Hp), dtype=np.float32)
    rb0 = rng.standard_normal((w.R, w.B, w.H, w.Hp), dtype=np.float32)

    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x))
    dy_nvs, _ = buf.dispatch(plan, dev_bf16(dy))          # combine bwd
    gh = dev(gh0)
    rb = dev(rb0)
    buf.expert_wgrad(plan, x_nvs, dy_nvs, gh, rb)
    torch.cuda.synchronize()
    gh1, rb1 = gh.cpu().numpy(), rb.cpu().numpy()

    xo, _ = oracle.dispatch(p, x)
    dyo, _ = oracle.dispatch(p, dy)
    gw, rw_ = oracle.expert_wgrad(p, xo, dyo, gh0, rb0)
    assert np.abs(gh1 - gw).max() <= 2e-2
    assert rel_l2(gh1 - gh0, gw - gh0) <= 1e-2
    assert np.abs(rb1 - rw_).max() <= 2e-2
    assert rel_l2(rb1 - rb0, rw_ - rb0) <= 1e-2

    # reduce_grad on identical inputs for all three projections
    log(f"reduce_grad {name} target={target}")
    ghs = [dev(gh1 + i) for i in range(3)]
    rbs = [dev(rb1 * (i + 1)) for i in range(3)]
    buf.reduce_grad(plan, ghs, rbs)
    torch.cuda.synchronize()
    for i in range(3):
        want_g, want_r = oracle.reduce_grad(p, (gh1 + i).astype(np.float32),
                                            (rb1 * (i + 1)).astype(np.float32))
        got_g, got_r = ghs[i].cpu().numpy(), rbs[i].cpu().numpy()
        assert np.abs(got_g - want_g).max() <= 1e-6 * max(np.abs(want_g).max(), 1.0)
        assert np.array_equal(got_r, want_r)
    buf.destroy()


@pytest.mark.parametrize("name,target", [("tiny_r4_s64_k2_e8", "adv"),
                                         ("bwd_r8_s1024_k4_e32", 2.0)])
def test_grads_equal_dense_expert_grads(name, target):
    w = synth.WORKLOADS[name]
    log(f"dense grads {name} target={target}")
    topk, _ = synth.routing(w, target)
    x = synth.hidden(w)
    dy = synth.grad_out(w, w.Hp)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x))
    dy_nvs, _ = buf.dispatch(plan, dev_bf16(dy))
    ghs = [torch.zeros((w.E, w.H, w.Hp), device="cuda") for _ in range(3)]
    rbs = [torch.zeros((w.R, w.B, w.H, w.Hp), device="cuda") for _ in range(3)]
    for i in range(3):
        buf.expert_wgrad(plan, x_nvs, dy_nvs, ghs[i], rbs[i])
    buf.reduce_grad(plan, ghs, rbs)
    torch.cuda.synchronize()
    ref = oracle.dense_expert_grad(topk, x, dy, w.E)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    assert p.dup_count > 0
    for i in range(3):
        g = ghs[i].cpu().numpy()
        assert np.abs(g - ref).max() <= 2e-2 and rel_l2(g, ref) <= 1e-2
        assert (rbs[i].cpu().numpy() == 0).all()
    buf.destroy()


@pytest.mark.parametrize("name,target", [("tiny_r4_s64_k2_e8", 1.0),
                                         ("bwd_r8_s1024_k4_e32", 2.0)])
def test_wgrad_per_rank_launches_equal_one_launch(name, target):
    """Each rank's weight gradients launched alone (rank = d, as with one GPU
    per rank) give, bit for bit, what one launch over all ranks gives: every
    output tile is computed the same way whichever launch enumerates it."""
    w = synth.WORKLOADS[name]
    log(f"wgrad per rank {name} target={target}")
    topk, _ = synth.routing(w, target)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(synth.hidden(w)))
    dy_nvs, _ = buf.dispatch(plan, dev_bf16(synth.grad_out(w, w.Hp)))
    rng = np.random.default_rng(5)
    gh0 = dev(rng.standard_normal((w.E, w.H, w.Hp), dtype=np.float32))
    rb0 = dev(rng.standard_normal((w.R, w.B, w.H, w.Hp), dtype=np.float32))
    gh_all, rb_all = gh0.clone(), rb0.clone()
    buf.expert_wgrad(plan, x_nvs, dy_nvs, gh_all, rb_all)
    gh_one, rb_one = gh0.clone(), rb0.clone()
    for d in range(w.R):
        buf.expert_wgrad(plan, x_nvs, dy_nvs, gh_one, rb_one, rank=d)
    torch.cuda.synchronize()
    assert not torch.equal(gh_all, gh0)
    assert torch.equal(gh_one, gh_all)
    assert torch.equal(rb_one, rb_all)
    buf.destroy()


def test_wgrad_full_size_sampled():
    """Headline shapes, all ranks in one launch, into zeroed gradient rows.
    A weight gradient separates over its output columns, so the oracle runs
    the whole plan on sampled columns of both operands (its own dispatch of
    the same inputs, restricted to those columns) and every home row and
    used slot is compared on those columns."""
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    log("wgrad full size")
    topk, _ = synth.routing(w, 2.0)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((w.R, w.S, w.H), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((w.R, w.S, w.Hp), generator=g, device="cuda").to(torch.bfloat16)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, x)
    b_nvs, _ = buf.dispatch(plan, b)
    gh = torch.zeros((w.E, w.H, w.Hp), device="cuda")
    rb = torch.zeros((w.R, w.B, w.H, w.Hp), device="cuda")
    buf.expert_wgrad(plan, x_nvs, b_nvs, gh, rb)
    torch.cuda.synchronize()
    del x_nvs, b_nvs
    rng = np.random.default_rng(12)
    hs = np.unique(np.concatenate([[0, w.H - 1], rng.choice(w.H, 46, replace=False)]))
    hps = np.unique(np.concatenate([[0, w.Hp - 1], rng.choice(w.Hp, 46, replace=False)]))
    hs_d = torch.from_numpy(hs).cuda()
    hps_d = torch.from_numpy(hps).cuda()
    got_h = gh.index_select(1, hs_d).index_select(2, hps_d).cpu().numpy()
    got_r = rb.index_select(2, hs_d).index_select(3, hps_d).cpu().numpy()
    xa, _ = oracle.dispatch(p, host_bf16(x)[:, :, hs])
    ba, _ = oracle.dispatch(p, host_bf16(b)[:, :, hps])
    want_h, want_r = oracle.expert_wgrad(p, xa, ba,
                                         np.zeros((w.E, len(hs), len(hps)), np.float32),
                                         np.zeros((w.R, w.B, len(hs), len(hps)), np.float32))
    assert np.abs(want_h).max() > 1.0 and np.abs(want_r).max() > 1.0
    assert np.abs(got_h - want_h).max() <= 2e-2 and rel_l2(got_h, want_h) <= 1e-2
    assert np.abs(got_r - want_r).max() <= 2e-2 and rel_l2(got_r, want_r) <= 1e-2
    buf.destroy()


def test_backward_data_path():
    """dispatch bwd (unweighted combine of a width-H gradient) against the
    oracle, bit for bit."""
    w = synth.WORKLOADS["bwd_r8_s1024_k4_e32"]
    topk, _ = synth.routing(w, 2.0)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    rng = np.random.default_rng(2)
    g_nvs = synth.to_bf16_bits(rng.standard_normal((w.R, p.NvS, w.H), dtype=np.float32))
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    out, _ = buf.combine(plan, dev_bf16(g_nvs))
    want, _ = oracle.combine(p, g_nvs, None)
    from gpu_util import host_bf16
    assert np.array_equal(host_bf16(out), want)
    buf.destroy()


def test_training_calls_need_full_prefetch():
    """B < E/R is inference only: the weight-gradient calls refuse it on the
    host with MOONEP_ERR_MODE before touching any buffer."""
    import ctypes
    from grouped_gemm_moonep_amd import _abi
    w = synth.WORKLOADS["infer_r8_s128_k8_e256_b4"]
    buf = buffer_for(w)
    plan = buf.new_plan()
    lib = _abi.lib()
    P3 = ctypes.c_void_p * 3
    dummy = P3(16, 16, 16)
    st = lib.moonep_reduce_grad(buf._h, ctypes.byref(plan.struct), dummy, dummy, None)
    assert st == _abi.MOONEP_ERR_MODE
    st = lib.moonep_expert_wgrad(buf._h, ctypes.byref(plan.struct), -1, 16, 16, 16, 16, None)
    assert st == _abi.MOONEP_ERR_MODE
    buf.destroy()
