"""Symmetric [E+B,H,H'] buffers on virtual memory (moonep_symbuf_*) on the
GPU: the README's weight and gradient buffer layout ("Usage > Integration >
Weight buffer", "Gradient buffer").

* every rank's view maps the same physical home chunks (a write through any
  range is read through every other range), and its rows [E,E+B) are its own
  slots;
* prefetch_weight_views fills rows [E,E+B) of each view from rows [0,E) of
  the same view, as the oracle's plan says (prefetch_src), bit for bit;
* the grouped FFN, forward and backward, over the views (experts located by
  row index only) matches the oracle's grouped FFN on host-drawn weights
  (forward and backward tolerances of the FFN tests) and is bit-identical to
  the same call over the symbuf's home/slots ranges and over ordinary device
  tensors; at the headline shape sampled rows are checked against the
  oracle's per-token FFN;
* an fp32 gradient symbuf takes the weight gradients and reduce_grad through
  its home and slots ranges, bit-identical to ordinary tensors, and its
  per-rank views show the reduce slots."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import assert_close_bf16, buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def same(a, b):
    return torch.equal(bits(a), bits(b))


def symbufs(buf, w, n=3, dtype=torch.bfloat16):
    from grouped_gemm_moonep_amd import SymmetricBuffer, vmm_granularity
    g = vmm_granularity()
    elem = 2 if dtype == torch.bfloat16 else 4
    row = w.H * w.Hp * elem
    if (w.E // w.R) * row % g or w.B * row % g:
        pytest.skip(f"{w.name}: chunks of {row} B rows are not multiples of the "
                    f"{g} B VMM granularity")
    log(f"symbuf {w.name} {dtype} granularity={g}")
    return [SymmetricBuffer(buf, dtype) for _ in range(n)]


def filled_weights(buf, w, host=None):
    """Three weight symbufs with the seeded expert weights in their home
    chunks (drawn on the GPU, or the host arrays `host` copied in) and a
    sentinel in every slot."""
    sbs = symbufs(buf, w)
    for i, sb in enumerate(sbs):
        if host is None:
            synth.expert_weights_device(w, i, sb.home)
        else:
            sb.home.copy_(dev_bf16(host[i]))
        bits(sb.slots).fill_(0x7F7F)
    return sbs


def test_views_alias_home_and_slots():
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    R, E, B, H, Hp = w.R, w.E, w.B, w.H, w.Hp
    buf = buffer_for(w)
    (sb,) = symbufs(buf, w, 1)
    assert sb.views.shape == (R, E + B, H, Hp)
    assert sb.home.shape == (E, H, Hp) and sb.slots.shape == (R, B, H, Hp)
    assert sb.physical_bytes == (E + R * B) * H * Hp * 2
    assert sb.row_bytes == H * Hp * 2
    synth.expert_weights_device(w, 0, sb.home)
    g = torch.Generator(device="cuda").manual_seed(5)
    sb.slots.copy_(torch.randn((R, B, H, Hp), generator=g, device="cuda").to(torch.bfloat16))
    torch.cuda.synchronize()
    for d in range(R):
        assert same(sb.views[d, :E], sb.home), d
        assert same(sb.views[d, E:], sb.slots[d]), d
    # a write through one rank's view is seen through the home range and every view
    before = sb.views[1, E + 1].clone()
    sb.views[3, 5].fill_(1.5)
    sb.views[2, E + 1].fill_(-2.0)
    torch.cuda.synchronize()
    assert bool((sb.home[5] == 1.5).all())
    for d in range(R):
        assert bool((sb.views[d, 5] == 1.5).all()), d
    assert bool((sb.slots[2, 1] == -2.0).all())
    assert same(sb.views[1, E + 1], before)          # other ranks' slots are their own
    del sb
    buf.destroy()


def test_layers_share_one_prefetch_pool():
    """Two layers' weight buffers mapping one set of slot chunks (the README's
    process-wide prefetch pool): a slot written through one layer's view is
    read through the other's, each layer keeps its own home rows, the second
    allocates only E rows, and the pool outlives the symbuf that created it."""
    from grouped_gemm_moonep_amd import SymmetricBuffer
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    E, B = w.E, w.B
    buf = buffer_for(w)
    (l0,) = symbufs(buf, w, 1)
    l1 = SymmetricBuffer(buf, slots_from=l0)
    assert l1.physical_bytes == E * l0.row_bytes
    assert l0.physical_bytes == (E + w.R * B) * l0.row_bytes
    l0.home.fill_(1.0)
    l1.home.fill_(2.0)
    l0.views[4, E + 2].fill_(3.0)
    torch.cuda.synchronize()
    assert bool((l1.views[4, E + 2] == 3.0).all()) and bool((l1.slots[4, 2] == 3.0).all())
    assert bool((l1.views[4, :E] == 2.0).all()) and bool((l0.views[4, :E] == 1.0).all())
    l0.destroy()
    l1.views[5, E + 3].fill_(4.0)
    torch.cuda.synchronize()
    assert bool((l1.slots[5, 3] == 4.0).all()) and bool((l1.views[4, E + 2] == 3.0).all())
    l1.destroy()
    from grouped_gemm_moonep_amd import MoonepError
    other = buffer_for(synth.WORKLOADS["tiny_r4_s64_k2_e8"])
    l2 = SymmetricBuffer(other)
    with pytest.raises(MoonepError):
        SymmetricBuffer(buf, slots_from=l2)          # another R, B and row size
    l2.destroy()
    other.destroy()
    buf.destroy()


@pytest.mark.parametrize("target", [2.0, "adv"])
def test_prefetch_views_matches_oracle_plan(target):
    w = synth.WORKLOADS["mid_r8_s1024_k4_e32"]
    log(f"prefetch views {w.name} target={target}")
    topk, _ = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    sbs = filled_weights(buf, w)
    buf.prefetch_weight_views(plan, [sb.views for sb in sbs])
    torch.cuda.synchronize()
    for i, sb in enumerate(sbs):
        for d in range(w.R):
            for j in range(w.B):
                e = p.prefetch_src[d, j]
                if e >= 0:
                    assert same(sb.views[d, w.E + j], sb.home[e]), (i, d, j)
                else:
                    assert bool((bits(sb.slots[d, j]) == 0x7F7F).all()), (i, d, j)
    del sbs
    buf.destroy()


@pytest.mark.parametrize("name,target", [("mid_r8_s1024_k4_e32", 2.0),
                                         ("mid_r8_s1024_k4_e32", "adv")])
def test_ffn_views_equal_split_and_plain(name, target):
    w = synth.WORKLOADS[name]
    log(f"ffn views {name} target={target}")
    topk, rw = synth.routing(w, target)
    x = synth.hidden(w)
    home_h = [synth.expert_weights_host(w, i) for i in range(3)]
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x), dev(rw))
    sbs = filled_weights(buf, w, home_h)
    views = [sb.views for sb in sbs]
    buf.prefetch_weight_views(plan, views)
    home_plain = [sb.home.clone() for sb in sbs]
    pool_plain = [sb.slots.clone() for sb in sbs]
    zeros = lambda: torch.zeros((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device="cuda")
    y_views, y_split, y_plain = zeros(), zeros(), zeros()
    buf.expert_ffn_views(plan, x_nvs, views, y_nvs=y_views)
    buf.expert_ffn(plan, x_nvs, [sb.home for sb in sbs], [sb.slots for sb in sbs], y_nvs=y_split)
    buf.expert_ffn(plan, x_nvs, home_plain, pool_plain, y_nvs=y_plain)
    torch.cuda.synchronize()
    assert bool((bits(y_views) != 0).any())
    assert same(y_views, y_split)
    assert same(y_views, y_plain)
    # the views path against the oracle's grouped FFN over the same plan
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs_h, _ = oracle.dispatch(p, x)
    pool_h = [oracle.prefetch_weight(p, home_h[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
              for i in range(3)]
    _, y_want = oracle.expert_ffn(p, x_nvs_h, home_h, pool_h)
    yv = host_bf16(y_views)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert_close_bf16(yv[d, :end], y_want[d, :end], what=f"views y rank {d}")
    # one rank at a time
    y_r = zeros()
    for d in range(w.R):
        buf.expert_ffn_views(plan, x_nvs, views, y_nvs=y_r, rank=d)
    torch.cuda.synchronize()
    assert same(y_r, y_views)
    del sbs, views
    buf.destroy()


def test_ffn_bwd_views_equal_plain():
    w = synth.WORKLOADS["bwd_r8_s1024_k4_e32"]
    log(f"ffn bwd views {w.name}")
    topk, rw = synth.routing(w, 2.0)
    x = synth.hidden(w)
    dout = synth.grad_out(w, w.H)
    home_h = [synth.expert_weights_host(w, i) for i in range(3)]
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(x))
    dy_nvs, _ = buf.dispatch(plan, dev_bf16(dout))
    sbs = filled_weights(buf, w, home_h)
    views = [sb.views for sb in sbs]
    buf.prefetch_weight_views(plan, views)
    home_plain = [sb.home.clone() for sb in sbs]
    pool_plain = [sb.slots.clone() for sb in sbs]

    def run(fn, *wts):
        outs = [torch.zeros((w.R, buf.NvS, W), dtype=torch.bfloat16, device="cuda")
                for W in (w.Hp, w.Hp, w.Hp, w.H)]
        fn(plan, x_nvs, dy_nvs, *wts, *outs)
        return outs

    a = run(buf.expert_ffn_bwd_views, views)
    b = run(buf.expert_ffn_bwd, home_plain, pool_plain)
    torch.cuda.synchronize()
    for k, (u, v) in enumerate(zip(a, b)):
        assert bool((bits(u) != 0).any()), k
        assert same(u, v), k
    # the views path against the oracle's grouped FFN backward
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs_h, _ = oracle.dispatch(p, x)
    dy_nvs_h, _ = oracle.dispatch(p, dout)
    pool_h = [oracle.prefetch_weight(p, home_h[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
              for i in range(3)]
    ranks = [0, 3, 6]
    want = oracle.expert_ffn_backward(p, x_nvs_h, dy_nvs_h, home_h, pool_h, ranks=ranks)
    for nm, g_, w_ in zip(("dz", "dg", "du", "dx"), a, want):
        gh = host_bf16(g_)
        for d in ranks:
            end = p.cu_seqlens[d, -1]
            assert_close_bf16(gh[d, :end], w_[d, :end], what=f"views {nm} rank {d}",
                              ulps=1 if nm == "dz" else 2)
    del sbs, views
    buf.destroy()


def test_gradient_symbuf_wgrad_and_reduce():
    w = synth.WORKLOADS["bwd_r8_s1024_k4_e32"]
    log(f"gradient symbuf {w.name}")
    topk, _ = synth.routing(w, 2.0)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(synth.hidden(w)))
    dg_nvs, _ = buf.dispatch(plan, dev_bf16(synth.grad_out(w, w.Hp)))
    gsb = symbufs(buf, w, 3, torch.float32)
    g = torch.Generator(device="cuda").manual_seed(9)
    for sb in gsb:
        sb.home.copy_(torch.randn(sb.home.shape, generator=g, device="cuda"))
        sb.slots.zero_()
    gh_plain = [sb.home.clone() for sb in gsb]
    rb_plain = [sb.slots.clone() for sb in gsb]
    for i in range(3):
        buf.expert_wgrad(plan, x_nvs, dg_nvs, gsb[i].home, gsb[i].slots)
        buf.expert_wgrad(plan, x_nvs, dg_nvs, gh_plain[i], rb_plain[i])
    torch.cuda.synchronize()
    used = plan.prefetch_src.cpu().numpy().reshape(w.R, w.B) >= 0
    assert used.any()
    for i in range(3):
        assert same(gsb[i].home, gh_plain[i]) and same(gsb[i].slots, rb_plain[i]), i
        for d in range(w.R):
            assert same(gsb[i].views[d, w.E:], gsb[i].slots[d]), (i, d)
            assert same(gsb[i].views[d, :w.E], gsb[i].home), (i, d)
    buf.reduce_grad(plan, [sb.home for sb in gsb], [sb.slots for sb in gsb])
    buf.reduce_grad(plan, gh_plain, rb_plain)
    torch.cuda.synchronize()
    for i in range(3):
        assert same(gsb[i].home, gh_plain[i]), i
        for d in range(w.R):
            for j in range(w.B):
                if used[d, j]:
                    assert bool((gsb[i].views[d, w.E + j] == 0).all()), (i, d, j)
    del gsb
    buf.destroy()


def test_ffn_views_full_size():
    """The headline shape: 8 views of 288 rows of 28 MiB per projection
    (63 GiB of address space each), row offsets past 2^32 elements."""
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    log(f"ffn views full size {w.name}")
    topk, rw = synth.routing(w, "adv")
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    x_nvs, _ = buf.dispatch(plan, dev_bf16(synth.hidden(w)), dev(rw))
    sbs = filled_weights(buf, w)
    views = [sb.views for sb in sbs]
    buf.prefetch_weight_views(plan, views)
    p = np.asarray(plan.prefetch_src.cpu()).reshape(w.R, w.B)
    for d in range(w.R):
        for j in np.nonzero(p[d] >= 0)[0][:2]:
            assert same(sbs[0].views[d, w.E + j], sbs[0].home[p[d, j]]), (d, j)
    y_views = torch.zeros((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device="cuda")
    y_split = torch.zeros_like(y_views)
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device="cuda")
    buf.expert_ffn_views(plan, x_nvs, views, z_ws=z, y_nvs=y_views)
    buf.expert_ffn(plan, x_nvs, [sb.home for sb in sbs], [sb.slots for sb in sbs], z_ws=z,
                   y_nvs=y_split)
    torch.cuda.synchronize()
    assert same(y_views, y_split)
    # sampled rows of every rank's prefetch rows (remote experts read through
    # the rank's own slots) and of a home row, against the oracle's per-token FFN
    po = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_h = synth.hidden(w)
    xs = x_h.reshape(-1, w.H)
    rng = np.random.default_rng(12)
    checked = 0
    for d in range(w.R):
        rows = [r for r in range(w.E + w.B) if po.seg_tokens[d, r] > 0]
        for row in (rows[0], rows[-1]):
            e = row if row < w.E else po.prefetch_src[d, row - w.E]
            end = po.cu_seqlens[d, row]
            start = end - po.seg_len[d, row]
            slots = start + rng.choice(po.seg_tokens[d, row], min(8, po.seg_tokens[d, row]),
                                       replace=False)
            toks = po.src[d, slots] // w.K
            wts = [host_bf16(sbs[i].views[d, row]) for i in range(3)]
            assert all(np.array_equal(wt, host_bf16(sbs[i].home[e])) for i, wt in enumerate(wts))
            _, yw = oracle.ffn_token(xs[toks], *wts)
            assert_close_bf16(host_bf16(y_views[d, slots]), yw, what=f"views y d={d} row={row}")
            checked += 1
    assert checked == 2 * w.R
    del sbs, views
    buf.destroy()
