"""Edge shapes of the grouped GEMMs on the GPU, against the oracle.

Hidden and FFN sizes that are not multiples of the tile widths (N-tiles of
128 and 256 columns cut short; K not a multiple of 256), token_padding 1
(segments of any length, so both a segment's short tail tile of at most 128
rows and a longer partial tile occur), a single rank, K = 1, one token per
rank and B = 0.  Each shape runs the grouped SwiGLU FFN, its backward and,
where B = E/R, the weight gradients, at balanced and skewed routing:

* FFN and backward: rel-L2 <= 1e-2 and element-wise max(2e-2, 1 ulp) (2 ulps
  for dG, dU, dX), rows past each rank's last segment untouched, padding
  rows zero;
* weight gradients: max-abs <= 2e-2 and rel-L2 <= 1e-2 on the increment."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import assert_close_bf16, buffer_for, dev, dev_bf16, host_bf16, log, rel_l2

pytestmark = pytest.mark.gpu

SENT = 0x7F7F

SHAPES = [
    synth.Workload("e_r1", R=1, S=100, K=3, E=8, B=8, H=192, Hp=320, token_padding=4),
    synth.Workload("e_k1", R=4, S=300, K=1, E=8, B=2, H=320, Hp=192, token_padding=8),
    synth.Workload("e_tp1", R=8, S=513, K=4, E=64, B=8, H=64, Hp=64, token_padding=1),
    synth.Workload("e_b0", R=4, S=257, K=2, E=16, B=0, H=128, Hp=128, token_padding=16),
    synth.Workload("e_s1", R=3, S=1, K=2, E=6, B=2, H=64, Hp=192, token_padding=2),
    synth.Workload("e_tails", R=2, S=700, K=2, E=4, B=2, H=448, Hp=320, token_padding=1),
    # padding granularities above the 128-row short tile: segment tails of any length
    synth.Workload("e_tp200", R=2, S=300, K=2, E=4, B=2, H=128, Hp=192, token_padding=200),
    synth.Workload("e_tp384", R=4, S=200, K=3, E=8, B=2, H=192, Hp=128, token_padding=384),
]


def _sent(shape):
    return torch.full(shape, SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _inputs(w, s):
    topk, rw = synth.routing_zipf(w, s, seed=7)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs, _ = oracle.dispatch(p, synth.hidden(w))
    dy_nvs, _ = oracle.dispatch(p, synth.grad_out(w, w.H))
    home = [synth.expert_weights_host(w, i) for i in range(3)]
    pool = [oracle.prefetch_weight(p, home[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
            for i in range(3)]
    return topk, p, x_nvs, dy_nvs, home, pool


def _device(buf, w, topk, home):
    plan = buf.plan(dev(topk))
    home_d = [dev_bf16(h) for h in home]
    pool_d = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
              for _ in range(3)]
    buf.prefetch_weight(plan, home_d, pool_d)
    return plan, home_d, pool_d


def _check_rows(p, w, got, want, what, ulps=1):
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        assert_close_bf16(got[d, :end], want[d, :end], what=f"{what} rank {d}", ulps=ulps)
        assert (got[d, end:] == SENT).all(), f"{what} rank {d} written past the last segment"


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
@pytest.mark.parametrize("s", [0.0, 1.5])
def test_edge_ffn_forward_and_backward(w, s):
    log(f"edge ffn {w.name} s={s}")
    topk, p, x_nvs, dy_nvs, home, pool = _inputs(w, s)
    z_want, y_want = oracle.expert_ffn(p, x_nvs, home, pool)
    bwd_want = oracle.expert_ffn_backward(p, x_nvs, dy_nvs, home, pool)
    buf = buffer_for(w)
    plan, home_d, pool_d = _device(buf, w, topk, home)
    x_d, dy_d = dev_bf16(x_nvs), dev_bf16(dy_nvs)
    z, y = _sent((w.R, buf.NvS, w.Hp)), _sent((w.R, buf.NvS, w.H))
    buf.expert_ffn(plan, x_d, home_d, pool_d, z, y)
    outs = [_sent((w.R, buf.NvS, W)) for W in (w.Hp, w.Hp, w.Hp, w.H)]
    buf.expert_ffn_bwd(plan, x_d, dy_d, home_d, pool_d, *outs)
    yg = host_bf16(y)
    _check_rows(p, w, host_bf16(z), z_want, "z")
    _check_rows(p, w, yg, y_want, "y")
    for nm, o, want in zip(("dz", "dg", "du", "dx"), outs, bwd_want):
        _check_rows(p, w, host_bf16(o), want, nm, ulps=1 if nm == "dz" else 2)
    for d in range(w.R):
        end = p.cu_seqlens[d, -1]
        pad = p.src[d, :end] < 0
        assert (yg[d, :end][pad] == 0).all()
    buf.destroy()


@pytest.mark.parametrize("w", [x for x in SHAPES if x.B == x.E // x.R],
                         ids=[x.name for x in SHAPES if x.B == x.E // x.R])
def test_edge_wgrad(w):
    log(f"edge wgrad {w.name}")
    topk, p, x_nvs, _, home, pool = _inputs(w, 1.5)
    b_nvs, _ = oracle.dispatch(p, synth.grad_out(w, w.Hp, stream_offset=1))
    rng = np.random.default_rng(3)
    gh0 = rng.standard_normal((w.E, w.H, w.Hp), dtype=np.float32)
    rb0 = rng.standard_normal((w.R, w.B, w.H, w.Hp), dtype=np.float32)
    gw, rw_ = oracle.expert_wgrad(p, x_nvs, b_nvs, gh0, rb0)
    buf = buffer_for(w)
    plan = buf.plan(dev(topk))
    gh, rb = dev(gh0), dev(rb0)
    buf.expert_wgrad(plan, dev_bf16(x_nvs), dev_bf16(b_nvs), gh, rb)
    gh1, rb1 = gh.cpu().numpy(), rb.cpu().numpy()
    assert np.abs(gh1 - gw).max() <= 2e-2
    assert rel_l2(gh1 - gh0, gw - gh0) <= 1e-2
    assert np.abs(rb1 - rw_).max() <= 2e-2
    if np.abs(rw_ - rb0).max() > 0:
        assert rel_l2(rb1 - rb0, rw_ - rb0) <= 1e-2
    buf.destroy()
