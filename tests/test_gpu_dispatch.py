"""moonep_dispatch on the GPU: bit copies of the token rows into their slots,
zero padding rows, route weights alongside; slots past a rank's last segment
untouched.  Checked against the oracle's dispatch of the same inputs."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F   # a finite bf16 pattern no generator produces here


def run(w, target, width=None, with_rw=True, num_cus=0):
    W = w.H if width is None else width
    log(f"dispatch {w.name} target={target} W={W} rw={with_rw} num_cus={num_cus}")
    topk, rw = synth.routing(w, target)
    x = synth.hidden(w, width=W)
    buf = buffer_for(w, num_cus=num_cus)
    plan = buf.plan(dev(topk))
    x_nvs = torch.full((w.R, buf.NvS, W), 0, dtype=torch.int16, device="cuda")
    x_nvs.fill_(SENTINEL)
    x_nvs = x_nvs.view(torch.bfloat16)
    rw_nvs = torch.full((w.R, buf.NvS), -7.0, dtype=torch.float32, device="cuda") if with_rw else None
    buf.dispatch(plan, dev_bf16(x), dev(rw) if with_rw else None, x_nvs=x_nvs, rw_nvs=rw_nvs)
    got = host_bf16(x_nvs)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    want, want_rw = oracle.dispatch(p, x, rw if with_rw else None)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert np.array_equal(got[d, :end], want[d, :end]), f"rank {d} rows"
        assert (got[d, end:] == SENTINEL).all(), f"rank {d} tail written"
        if with_rw:
            grw = rw_nvs[d].cpu().numpy()
            assert np.array_equal(grw[:end].view(np.uint32), want_rw[d, :end].view(np.uint32))
            assert (grw[end:] == -7.0).all()
    buf.destroy()


@pytest.mark.parametrize("name,target", [
    (n, t) for n, ts in synth.SWEEPS.items() for t in ts
    if n.startswith(("tiny", "mid", "infer"))])
def test_dispatch_matches_oracle(name, target):
    run(synth.WORKLOADS[name], target)


def test_dispatch_gradient_width():
    """combine bwd: the output gradient of width H' dispatched with the plan."""
    w = synth.WORKLOADS["bwd_r8_s1024_k4_e32"]
    run(w, 2.0, width=w.Hp, with_rw=False)


@pytest.mark.parametrize("width", [8, 24, 520, 1032])
def test_dispatch_ragged_widths(width):
    run(synth.WORKLOADS["tiny_r4_s64_k2_e8"], "adv", width=width)


@pytest.mark.parametrize("name,num_cus", [("mid_r8_s1024_k4_e32", 4), ("tiny_r4_s64_k2_e8", 1)])
def test_dispatch_cu_budget(name, num_cus):
    """A CU budget caps the whole dispatch grid (num_cus * 8 workgroups, here
    down to 8): every workgroup loops over the padding items, then over the
    token items."""
    run(synth.WORKLOADS[name], 1.0, num_cus=num_cus)


@pytest.mark.parametrize("name,target", [("fwd_r8_s4096_k8_e256", 2.0),
                                         ("pages_r8_s8192_k8_e384", 20.0)])
def test_dispatch_full_size_sampled(name, target):
    """Full size (4.7 GB of slots at the headline, 8.9 GB at the pages' shape):
    sampled slots checked through the oracle's src map; padding rows sampled
    for zeros."""
    w = synth.WORKLOADS[name]
    topk, rw = synth.routing(w, target)
    log(f"dispatch {name} maxvio={target}")
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((w.R, w.S, w.H), generator=g, device="cuda").to(torch.bfloat16)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, rw_nvs = buf.dispatch(plan, x, dev(rw))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    d = rng.integers(0, w.R, 4096)
    slot = np.minimum(rng.integers(0, buf.NvS, 4096), p.cu_seqlens[d, -1] - 1)
    src = p.src[d, slot]
    real = src >= 0
    tok = src[real] // w.K
    got_rows = host_bf16(x_nvs[torch.from_numpy(d[real]).cuda(), torch.from_numpy(slot[real]).cuda()])
    want_rows = host_bf16(x.reshape(-1, w.H)[torch.from_numpy(tok).cuda()])
    assert np.array_equal(got_rows, want_rows)
    pad_rows = host_bf16(x_nvs[torch.from_numpy(d[~real]).cuda(), torch.from_numpy(slot[~real]).cuda()])
    assert (pad_rows == 0).all()
    grw = rw_nvs.cpu().numpy()
    assert np.array_equal(grw[d[real], slot[real]], rw.reshape(-1)[src[real]])
    buf.destroy()


@pytest.mark.parametrize("target", [1.0, "adv"])
def test_copy_mode_equals_zero_copy(target):
    """zero_copy=False (README "API guide > zero_copy"): dispatch into the
    Buffer's communication buffer and copy the used slots out; combine copies
    its input in first.  Same bits as the zero-copy calls and as the oracle's
    dispatch and combine on every used slot; rows past the last segment of the
    destination are left alone."""
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    topk, rw = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x = dev_bf16(synth.hidden(w))
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    a, ra = buf.dispatch(plan, x, dev(rw))
    b = torch.full((w.R, buf.NvS, w.H), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    b, rb = buf.dispatch(plan, x, dev(rw), x_nvs=b, zero_copy=False)
    ah, bh = host_bf16(a), host_bf16(b)
    rah, rbh = ra.cpu().numpy().view(np.uint32), rb.cpu().numpy().view(np.uint32)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert np.array_equal(ah[d, :end], bh[d, :end])
        assert (bh[d, end:] == SENTINEL).all()
        # rw_nvs past the last segment is not written by either call
        assert np.array_equal(rah[d, :end], rbh[d, :end])
    # both modes against the oracle's dispatch of the same inputs
    want, want_rw = oracle.dispatch(p, synth.hidden(w), rw)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert np.array_equal(bh[d, :end], want[d, :end]), f"copy mode rank {d} rows"
        assert np.array_equal(rbh[d, :end], want_rw[d, :end].view(np.uint32)), f"rank {d} rw"
    o1, g1 = buf.combine(plan, a, ra)
    o2, g2 = buf.combine(plan, b, rb, zero_copy=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(g1, g2)
    # copy-mode combine of the copy-mode dispatch against the oracle's combine
    out_want, rw_want = oracle.combine(p, want, want_rw)
    assert np.array_equal(host_bf16(o2), out_want)
    assert np.array_equal(g2.cpu().numpy().view(np.uint32), rw_want.view(np.uint32))
    buf.destroy()
