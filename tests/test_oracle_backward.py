"""Pins for the oracle's SwiGLU backward (oracle/swiglu.py) and its grouped
form over a plan (oracle.expert_ffn_backward).

* finite differences: with no rounding, dX, X^T dG, X^T dU, dY^T Z and dZ are
  the central-difference derivatives of L = sum(dY * Y) with respect to X, Wg,
  Wu, Wd and Z (float64, several shapes);
* the rounded forward in swiglu.forward equals the independently written
  oracle.ffn_token bit for bit;
* the grouped backward over a plan's segments equals the per-token backward
  of the token in each slot, with zero rows at padding slots;
* zero gradient in, zero gradient out.
"""
import numpy as np
import pytest

import moonep_synth as synth
import oracle
from oracle import swiglu


def _loss(x, dy, wg, wu, wd):
    return float(np.sum(dy * swiglu.forward(x, wg, wu, wd)[1]))


def _fd(f, v, eps=1e-6):
    g = np.zeros_like(v)
    it = np.nditer(v, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = v[i]
        v[i] = old + eps
        fp = f()
        v[i] = old - eps
        fm = f()
        v[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("n,H,Hp,seed", [(1, 1, 1, 0), (3, 4, 3, 1), (5, 6, 8, 2), (2, 8, 5, 3)])
def test_backward_matches_finite_differences(n, H, Hp, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, H))
    dy = rng.standard_normal((n, H))
    wg, wu, wd = (rng.standard_normal((H, Hp)) * 0.7 for _ in range(3))
    dz, dg, du, dx = swiglu.backward(x, dy, wg, wu, wd)
    z, _ = swiglu.forward(x, wg, wu, wd)
    f = lambda: _loss(x, dy, wg, wu, wd)
    np.testing.assert_allclose(dx, _fd(f, x), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(x.T @ dg, _fd(f, wg), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(x.T @ du, _fd(f, wu), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dy.T @ z, _fd(f, wd), rtol=1e-6, atol=1e-7)
    # dZ: derivative of sum(dY * (Z Wd^T)) with respect to Z
    zz = z.copy()
    np.testing.assert_allclose(dz, _fd(lambda: float(np.sum(dy * (zz @ wd.T))), zz),
                               rtol=1e-6, atol=1e-7)


def test_rounded_forward_equals_ffn_token():
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    x = synth.hidden(w).reshape(-1, w.H)[:40]
    home = [synth.expert_weights_host(w, i) for i in range(3)]
    f = lambda b: oracle.bf16_to_f32(b).astype(np.float64)
    rnd = lambda v: oracle.bf16_to_f32(oracle.f64_to_bf16(v)).astype(np.float64)
    e = 3
    z, y = swiglu.forward(f(x), f(home[0][e]), f(home[1][e]), f(home[2][e]), rnd=rnd)
    z_ref, y_ref = oracle.ffn_token(x, home[0][e], home[1][e], home[2][e])
    assert np.array_equal(oracle.f64_to_bf16(z), z_ref)
    assert np.array_equal(oracle.f64_to_bf16(y), y_ref)


def _dy_nvs(plan, W, seed):
    """Seeded gradient rows for the slots that hold a token, zero at padding
    (as a dispatch of a token-major gradient leaves them)."""
    rng = np.random.default_rng(seed)
    dy = oracle.f32_to_bf16(rng.standard_normal((plan.R, plan.NvS, W)).astype(np.float32))
    dy[plan.src < 0] = 0
    return dy


@pytest.mark.parametrize("target", [1.0, "adv"])
def test_grouped_backward_equals_per_token(target):
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    topk, _ = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs, _ = oracle.dispatch(p, synth.hidden(w))
    dy_nvs = _dy_nvs(p, w.H, 5)
    home = [synth.expert_weights_host(w, i) for i in range(3)]
    pool = [oracle.prefetch_weight(p, home[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
            for i in range(3)]
    dz, dg, du, dx = oracle.expert_ffn_backward(p, x_nvs, dy_nvs, home, pool)
    for d in range(w.R):
        for row in range(w.E + w.B):
            n = p.seg_len[d, row]
            if n == 0:
                continue
            hi = p.cu_seqlens[d, row]
            lo = hi - n
            e = row if row < w.E else p.prefetch_src[d, row - w.E]
            want = oracle.ffn_token_backward(x_nvs[d, lo:hi], dy_nvs[d, lo:hi],
                                             home[0][e], home[1][e], home[2][e])
            for got, ref in zip((dz, dg, du, dx), want):
                assert np.array_equal(got[d, lo:hi], ref)
            pad = p.src[d, lo:hi] < 0
            assert (dx[d, lo:hi][pad] == 0).all() and (dg[d, lo:hi][pad] == 0).all()
    outside = np.ones((w.R, p.NvS), bool)
    for d in range(w.R):
        outside[d, :p.cu_seqlens[d, -1]] = False
    assert (dx[outside] == 0).all()


def test_zero_gradient_gives_zero():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 6))
    ws = [rng.standard_normal((6, 5)) for _ in range(3)]
    for v in swiglu.backward(x, np.zeros((4, 6)), *ws):
        assert not v.any()
