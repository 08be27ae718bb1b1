"""Pins for the oracle's data path: dispatch, combine, prefetch, the SwiGLU
FFN, weight gradients and reduce_grad.

* unweighted combine of a dispatch gives K*x exactly (K a power of two);
  gathered route weights come back bit-identical; padding rows are zero;
* prefetch rows equal their home rows;
* the SwiGLU formula against scipy's logistic function and hand values;
* combine(FFN(dispatch(x))) equals a dense per-token MoE that never sees the
  plan (<= 1 bf16 ulp, float64 product blocking only);
* weight gradients + reduce_grad equal dense per-expert gradients (float64,
  1e-6 relative) and leave every used reduce slot at zero;
* combine arithmetic against a pure-Python fp32 loop on a tiny case.
"""
import numpy as np
import pytest
from scipy.special import expit

import moonep_synth as synth
import oracle

TINY = synth.WORKLOADS["tiny_r4_s64_k2_e8"]


def _tiny_inputs(target=1.0, seed=0):
    w = TINY
    topk, rw = synth.routing(w, target, seed)
    x = synth.hidden(w, seed)
    home = [synth.expert_weights_host(w, p, seed) for p in range(3)]
    return w, topk, rw, x, home


@pytest.mark.parametrize("target", [0.0, 1.0, "adv"])
def test_dispatch_combine_roundtrip(target):
    w, topk, rw, x, _ = _tiny_inputs(target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs, rw_nvs = oracle.dispatch(p, x, rw)
    out, g = oracle.combine(p, x_nvs, None)
    assert g is None
    want = oracle.f32_to_bf16(oracle.bf16_to_f32(x) * np.float32(w.K))
    assert (out == want).all()
    _, g = oracle.combine(p, x_nvs, rw_nvs)
    assert (g.view(np.uint32) == rw.view(np.uint32)).all()
    # padding rows and route weights are zero; real rows are the token rows
    pad = p.src < 0
    assert (x_nvs[pad] == 0).all() and (rw_nvs[pad] == 0).all()
    d, slot = np.nonzero(~pad)
    t = p.src[d, slot]
    r, s, k = t // (w.S * w.K), (t // w.K) % w.S, t % w.K
    assert (x_nvs[d, slot] == x[r, s]).all()
    assert (rw_nvs[d, slot] == rw[r, s, k]).all()


def test_combine_matches_scalar_loop():
    w, topk, rw, x, _ = _tiny_inputs()
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    rng = np.random.default_rng(9)
    y = synth.to_bf16_bits(rng.standard_normal((w.R, p.NvS, 8), dtype=np.float32))
    rw_nvs = rng.random((w.R, p.NvS), dtype=np.float32)
    out, _ = oracle.combine(p, y, rw_nvs)
    yf = oracle.bf16_to_f32(y).reshape(-1, 8)
    for r in range(w.R):
        for s in range(0, w.S, 7):
            for c in range(8):
                acc = None
                for k in range(w.K):
                    slot = p.dest[r, s, k]
                    prod = np.float32(rw_nvs.reshape(-1)[slot]) * np.float32(yf[slot, c])
                    acc = prod if acc is None else np.float32(acc + prod)
                assert oracle.f32_to_bf16(np.array([acc], np.float32))[0] == out[r, s, c]


def test_prefetch_rows_equal_home_rows():
    w, topk, rw, x, home = _tiny_inputs()
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    assert (p.prefetch_src >= 0).any()
    pool0 = np.full((w.R, w.B, w.H, w.Hp), 0x7F7F, dtype=np.uint16)
    pool = oracle.prefetch_weight(p, home[0], pool0)
    for d in range(w.R):
        for j in range(w.B):
            e = p.prefetch_src[d, j]
            if e >= 0:
                assert (pool[d, j] == home[0][e]).all()
            else:
                assert (pool[d, j] == 0x7F7F).all()


def test_swiglu_formula_hand_values():
    # H = 2, H' = 2: x = [1, 0] picks row 0 of every projection
    bf = oracle.f32_to_bf16
    x = bf(np.array([1.0, 0.0], np.float32))
    wg = bf(np.array([[2.0, -1.0], [5.0, 5.0]], np.float32))
    wu = bf(np.array([[0.5, 3.0], [7.0, 7.0]], np.float32))
    wd = bf(np.array([[1.0, 0.0], [1.0, 1.0]], np.float32))   # [H, H']
    z, y = oracle.ffn_token(x, wg, wu, wd)
    g = np.array([2.0, -1.0])
    u = np.array([0.5, 3.0])
    zf = g * expit(g) * u                                      # silu(g) * u
    assert (z == oracle.f64_to_bf16(zf)).all()
    zb = oracle.bf16_to_f32(z).astype(np.float64)
    assert (y == oracle.f64_to_bf16(np.array([zb[0], zb[0] + zb[1]]))).all()


def test_silu_matches_logistic_on_grid():
    rng = np.random.default_rng(1)
    H, Hp = 16, 8
    bf = lambda a: synth.to_bf16_bits(a.astype(np.float32))
    x = bf(rng.standard_normal((5, H)))
    wg, wu, wd = (bf(rng.standard_normal((H, Hp)) * 0.5) for _ in range(3))
    z, y = oracle.ffn_token(x, wg, wu, wd)
    f = lambda b: oracle.bf16_to_f32(b).astype(np.float64)
    g = f(x) @ f(wg)
    u = f(x) @ f(wu)
    assert (z == oracle.f64_to_bf16(g * expit(g) * u)).all()
    assert (y == oracle.f64_to_bf16(f(z) @ f(wd).T)).all()


def _ulp_diff(a, b):
    fa = oracle.bf16_to_f32(a).astype(np.float64)
    fb = oracle.bf16_to_f32(b).astype(np.float64)
    ulp = np.abs(oracle.bf16_to_f32(a | 1) - oracle.bf16_to_f32(a & 0xFFFE)).astype(np.float64)
    ulp = np.maximum(ulp, 2.0 ** -133)
    return np.abs(fa - fb) / ulp


@pytest.mark.parametrize("target", [0.0, 1.0, "adv"])
def test_e2e_equals_dense_moe(target):
    w, topk, rw, x, home = _tiny_inputs(target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    x_nvs, rw_nvs = oracle.dispatch(p, x, rw)
    pool = [oracle.prefetch_weight(p, home[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
            for i in range(3)]
    z, y = oracle.expert_ffn(p, x_nvs, home, pool)
    out, _ = oracle.combine(p, y, rw_nvs)
    ref = oracle.dense_moe(topk, rw, x, home)
    diff = _ulp_diff(out, ref)
    assert diff.max() <= 1.0
    assert (diff == 0).mean() > 0.99
    # padding rows produce zero output
    assert (y[p.src < 0] == 0).all() and (z[p.src < 0] == 0).all()


def test_e2e_inference_overflow_rows():
    """B < E/R: remote experts beyond B run from their home rows; the result
    is unchanged (README "How to set B")."""
    w = synth.Workload("t", R=4, S=32, K=2, E=16, B=1, H=32, Hp=64, token_padding=4)
    topk, rw = synth.routing_zipf(w, 1.5)
    x = synth.hidden(w)
    home = [synth.expert_weights_host(w, p) for p in range(3)]
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    assert max(len(r) for r in p.remote_experts) > w.B       # overflow happens
    x_nvs, rw_nvs = oracle.dispatch(p, x, rw)
    pool = [oracle.prefetch_weight(p, home[i], np.zeros((w.R, w.B, w.H, w.Hp), np.uint16))
            for i in range(3)]
    _, y = oracle.expert_ffn(p, x_nvs, home, pool)
    out, _ = oracle.combine(p, y, rw_nvs)
    assert _ulp_diff(out, oracle.dense_moe(topk, rw, x, home)).max() <= 1.0


@pytest.mark.parametrize("target", [0.0, 1.0, "adv"])
def test_grads_equal_dense_expert_grads(target):
    w, topk, rw, x, _ = _tiny_inputs(target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    dy = synth.grad_out(w, w.Hp)
    x_nvs, _ = oracle.dispatch(p, x)
    dy_nvs, _ = oracle.dispatch(p, dy)
    gh0 = np.zeros((w.E, w.H, w.Hp), np.float32)
    rb0 = np.zeros((w.R, w.B, w.H, w.Hp), np.float32)
    gh, rb = oracle.expert_wgrad(p, x_nvs, dy_nvs, gh0, rb0)
    gh2, rb2 = oracle.reduce_grad(p, gh, rb)
    ref = oracle.dense_expert_grad(topk, x, dy, w.E)
    scale = np.abs(ref).max()
    assert np.abs(gh2 - ref).max() <= 1e-6 * scale
    for d in range(w.R):
        for j in range(w.B):
            if p.prefetch_src[d, j] >= 0:
                assert (rb2[d, j] == 0).all()
    if target == "adv":
        assert (p.prefetch_src >= 0).sum() > 0


def test_reduce_grad_order_is_ascending_rank():
    """Three ranks hold a duplicate of one expert: the fp32 sum must be
    ((home + slot_d0) + slot_d1) + slot_d2 with d0 < d1 < d2."""
    counts = [[8, 0, 0, 0], [8, 0, 0, 0], [8, 0, 0, 0], [8, 0, 0, 0]]
    topk = np.zeros((4, 8, 1), np.int32)
    p = oracle.plan(topk, E=4, B=1, token_padding=1)
    assert sorted(p.prefetch_src[:, 0].tolist()) == [-1, 0, 0, 0]
    big, tiny = np.float32(2.0 ** 24), np.float32(1.0)
    gh = np.full((4, 1, 1), big, np.float32)
    rb = np.zeros((4, 1, 1, 1), np.float32)
    rb[1], rb[2], rb[3] = tiny, tiny, -big
    gh2, rb2 = oracle.reduce_grad(p, gh, rb)
    # 2^24 + 1 rounds to 2^24 (even), twice; then - 2^24 -> 0
    assert gh2[0, 0, 0] == 0.0
    assert (rb2 == 0).all()
    del counts


def test_wgrad_rejects_inference_mode():
    w = synth.Workload("t", R=2, S=4, K=1, E=4, B=1, H=8, Hp=8, token_padding=1)
    topk = np.zeros((2, 4, 1), np.int32)
    p = oracle.plan(topk, w.E, w.B, 1)
    with pytest.raises(ValueError):
        oracle.expert_wgrad(p, np.zeros((2, p.NvS, 8), np.uint16),
                            np.zeros((2, p.NvS, 8), np.uint16),
                            np.zeros((4, 8, 8), np.float32), np.zeros((2, 1, 8, 8), np.float32))


def test_wgrad_accumulates():
    """Gradient rows accumulate across micro-batches (the reduce slots are
    zeroed for the next micro-batch, so writes add into them)."""
    w, topk, rw, x, _ = _tiny_inputs("adv")
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    dy = synth.grad_out(w, w.Hp)
    x_nvs, _ = oracle.dispatch(p, x)
    dy_nvs, _ = oracle.dispatch(p, dy)
    rng = np.random.default_rng(3)
    gh0 = rng.standard_normal((w.E, w.H, w.Hp)).astype(np.float32)
    rb0 = rng.standard_normal((w.R, w.B, w.H, w.Hp)).astype(np.float32)
    gh, rb = oracle.expert_wgrad(p, x_nvs, dy_nvs, gh0, rb0)
    ghz, rbz = oracle.expert_wgrad(p, x_nvs, dy_nvs, np.zeros_like(gh0), np.zeros_like(rb0))
    scale = np.abs(ghz).max()
    assert np.abs(gh - (gh0.astype(np.float64) + ghz)).max() <= 1e-6 * scale
    assert np.abs(rb - (rb0.astype(np.float64) + rbz)).max() <= 1e-6 * scale
