"""moonep_combine on the GPU: bit-exact against the oracle's combine when
both get the same expert outputs (weighted and unweighted), gathered route
weights bit-exact, and the dispatch-bwd identity combine(dispatch(x)) = K x."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu


def run(w, target, weighted=True, width=None, num_cus=0):
    W = w.H if width is None else width
    log(f"combine {w.name} target={target} W={W} weighted={weighted}")
    topk, rw = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    rng = np.random.default_rng(42)
    y = synth.to_bf16_bits(rng.standard_normal((w.R, p.NvS, W), dtype=np.float32))
    rw_nvs = rng.random((w.R, p.NvS), dtype=np.float32) if weighted else None
    buf = buffer_for(w, num_cus=num_cus)
    plan = buf.plan(dev(topk))
    out, rw_sk = buf.combine(plan, dev_bf16(y), dev(rw_nvs) if weighted else None)
    want, want_rw = oracle.combine(p, y, rw_nvs)
    assert np.array_equal(host_bf16(out), want)
    if weighted:
        assert np.array_equal(rw_sk.cpu().numpy().view(np.uint32), want_rw.view(np.uint32))
    else:
        assert rw_sk is None
    buf.destroy()


@pytest.mark.parametrize("name,target", [
    (n, t) for n, ts in synth.SWEEPS.items() for t in ts
    if n.startswith(("tiny", "mid", "infer"))])
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_matches_oracle(name, target, weighted):
    run(synth.WORKLOADS[name], target, weighted)


@pytest.mark.parametrize("width", [8, 40, 1032])
def test_combine_ragged_widths(width):
    run(synth.WORKLOADS["tiny_r4_s64_k2_e8"], 1.0, True, width=width)


def test_combine_cu_budget():
    run(synth.WORKLOADS["mid_r8_s1024_k4_e32"], 2.0, True, num_cus=3)


@pytest.mark.parametrize("target", [0.0, 1.0, "adv"])
def test_dispatch_bwd_identity(target):
    """dispatch bwd = unweighted combine: the K copies of x sum to K*x."""
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    topk, _ = synth.routing(w, target)
    x = synth.hidden(w)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x))
    out, _ = buf.combine(plan, x_nvs)
    want = oracle.f32_to_bf16(oracle.bf16_to_f32(x) * np.float32(w.K))
    assert np.array_equal(host_bf16(out), want)
    buf.destroy()


@pytest.mark.parametrize("name,target", [("fwd_r8_s4096_k8_e256", 4.0),
                                         ("pages_r8_s8192_k8_e384", 10.0)])
def test_combine_full_size_sampled(name, target):
    w = synth.WORKLOADS[name]
    topk, _ = synth.routing(w, target)
    log(f"combine {name} maxvio={target}")
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    g = torch.Generator(device="cuda").manual_seed(5)
    y = torch.randn((w.R, p.NvS, w.H), generator=g, device="cuda").to(torch.bfloat16)
    rw_nvs = torch.rand((w.R, p.NvS), generator=g, device="cuda")
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    out, rw_sk = buf.combine(plan, y, rw_nvs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    toks = rng.choice(w.R * w.S, 512, replace=False)
    slots = p.dest.reshape(-1, w.K)[toks]                       # [512, K]
    ys = host_bf16(y.reshape(-1, w.H)[torch.from_numpy(slots.reshape(-1)).cuda()])
    ws = rw_nvs.reshape(-1)[torch.from_numpy(slots.reshape(-1)).cuda()].cpu().numpy()
    ys = ys.reshape(512, w.K, w.H)
    ws = ws.reshape(512, w.K)
    want = oracle.combine_rows(ys, ws)
    got = host_bf16(out.reshape(-1, w.H)[torch.from_numpy(toks).cuda()])
    assert np.array_equal(got, want)
    assert np.array_equal(rw_sk.reshape(-1, w.K)[torch.from_numpy(toks).cuda()].cpu().numpy(), ws)
    buf.destroy()
