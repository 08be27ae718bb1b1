"""Dispatch, prefetch, grouped SwiGLU FFN, combine, weight gradients and
reduce_grad over a plan.  TEST INFRASTRUCTURE ONLY.

Sources (MoonEP README, MoonshotAI/MoonEP mirror):
* "API guide > dispatch fwd": hidden [S,H] bf16 and route weights [S,K] fp32
  go to hidden_nvsh [NvS,H] bf16 and route_weights_nvs [NvS] fp32 in the
  physical row order of the [E+B] weight tensor.
* "API guide > combine fwd": the K copies of a token come back to token-major
  order, optionally weighted by route_weights_nvs; gathered route weights
  [S,K] are returned as well.
* "API guide > combine bwd / dispatch bwd": the backward of combine is a
  re-dispatch with the saved plan; the backward of dispatch is an unweighted
  combine that sums the K copies.
* "Weight buffer": rows [0,E) of the [E+B,H,H'] tensor are home experts,
  rows [E,E+B) are prefetch slots filled by prefetch_weight.
* "Gradient buffer": fp32 [E+B,H,H'] gradients; rows [E,E+B) are backed by a
  per-rank reduce buffer, seen by all ranks as [R,B,H,H']; reduce_grad adds
  each rank's slots into the owning home rows and zeroes them.

Readings where the pages are silent (each is also listed in the design notes):
* rows inside a segment that hold no token (padding) are zero, route weight 0;
  slots past the last segment are left alone by the GPU and are 0 here;
* the FFN is SwiGLU: Z = bf16(silu(X Wg) * (X Wu)), Y = bf16(Z Wd^T), every
  projection stored [H,H'] (products in float64 here);
* combine: acc = p_0, then acc = fp32(acc + p_k) for k = 1..K-1 with
  p_k = fp32(w_k * y_k) (weighted) or y_k (unweighted), output bf16(acc);
* weight gradients accumulate (+=) in fp32; reduce_grad adds in ascending
  source rank in fp32.
"""
import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16, f64_to_bf16
from . import swiglu


def _token_of(plan, t):
    S, K = plan.S, plan.K
    return t // (S * K), (t // K) % S, t % K


def dispatch(plan, x: np.ndarray, rw=None):
    """x [R,S,W] bf16 bits -> x_nvs [R,NvS,W]; rw [R,S,K] -> rw_nvs [R,NvS]."""
    R, NvS = plan.R, plan.NvS
    W = x.shape[-1]
    x_nvs = np.zeros((R, NvS, W), dtype=np.uint16)
    rw_nvs = np.zeros((R, NvS), dtype=np.float32) if rw is not None else None
    d_idx, slot = np.nonzero(plan.src >= 0)
    r, s, k = _token_of(plan, plan.src[d_idx, slot])
    x_nvs[d_idx, slot] = x[r, s]
    if rw is not None:
        rw_nvs[d_idx, slot] = rw[r, s, k]
    return x_nvs, rw_nvs


def combine_rows(y_k: np.ndarray, w_k=None) -> np.ndarray:
    """The per-token combine sum: y_k [..., K, W] bf16 bits, w_k [..., K]
    fp32 or None -> [..., W] bf16 bits."""
    K = y_k.shape[-2]
    acc = None
    for k in range(K):
        yk = bf16_to_f32(y_k[..., k, :])
        if w_k is not None:
            pk = (np.asarray(w_k[..., k:k + 1], np.float32) * yk).astype(np.float32)
        else:
            pk = yk
        acc = pk if acc is None else (acc + pk).astype(np.float32)
    return f32_to_bf16(acc)


def combine(plan, y_nvs: np.ndarray, rw_nvs=None):
    """y_nvs [R,NvS,W] bf16 bits -> out [R,S,W] bf16 bits (+ gathered rw)."""
    R, NvS = plan.R, plan.NvS
    W = y_nvs.shape[-1]
    flat = y_nvs.reshape(R * NvS, W)
    y_k = flat[plan.dest]                                      # [R,S,K,W]
    w_k = rw_nvs.reshape(-1)[plan.dest] if rw_nvs is not None else None
    out = combine_rows(y_k, w_k)
    gathered = None
    if rw_nvs is not None:
        gathered = rw_nvs.reshape(-1)[plan.dest].astype(np.float32)
    return out, gathered


def prefetch_weight(plan, home: np.ndarray, pool: np.ndarray) -> np.ndarray:
    """pool[d][j] <- home[prefetch_src[d][j]] for every used slot."""
    pool = pool.copy()
    for d in range(plan.R):
        for j in range(plan.B):
            e = plan.prefetch_src[d, j]
            if e >= 0:
                pool[d, j] = home[e]
    return pool


def resolve_row(plan, d: int, row: int, home, pool):
    """Row `row` of rank d's [E+B] view: home rows below E, else the rank's
    own prefetch slot row-E."""
    if row < plan.E:
        return home[row]
    return pool[d, row - plan.E]


def _segments(plan, d):
    for row in range(plan.E + plan.B):
        ln = plan.seg_len[d, row]
        if ln > 0:
            end = plan.cu_seqlens[d, row]
            yield row, end - ln, end


def expert_ffn(plan, x_nvs, home, pool, ranks=None):
    """Grouped SwiGLU over every segment.  home = (gate, up, down) each
    [E,H,H'] bf16 bits; pool likewise [R,B,H,H'].  Returns z [R,NvS,H'] and
    y [R,NvS,H] bf16 bits (zero outside segments)."""
    R, NvS = plan.R, plan.NvS
    H = x_nvs.shape[-1]
    Hp = home[0].shape[-1]
    z = np.zeros((R, NvS, Hp), dtype=np.uint16)
    y = np.zeros((R, NvS, H), dtype=np.uint16)
    for d in (range(R) if ranks is None else ranks):
        for row, lo, hi in _segments(plan, d):
            X = bf16_to_f32(x_nvs[d, lo:hi]).astype(np.float64)
            wg, wu, wd = (bf16_to_f32(resolve_row(plan, d, row, home[p], pool[p]))
                          .astype(np.float64) for p in range(3))
            G = X @ wg
            U = X @ wu
            Zb = f64_to_bf16(G / (1.0 + np.exp(-G)) * U)
            Y = bf16_to_f32(Zb).astype(np.float64) @ wd.T
            z[d, lo:hi] = Zb
            y[d, lo:hi] = f64_to_bf16(Y)
    return z, y


def expert_ffn_backward(plan, x_nvs, dy_nvs, home, pool, ranks=None):
    """Backward of the grouped SwiGLU over every segment (swiglu.backward,
    stored tensors rounded to bf16): x_nvs, dy_nvs [R,NvS,H] bf16 bits ->
    dz, dg, du [R,NvS,H'] and dx [R,NvS,H] bf16 bits, zero outside segments.
    dy_nvs is the gradient of the loss w.r.t. the FFN output rows y_nvs."""
    R, NvS = plan.R, plan.NvS
    H = x_nvs.shape[-1]
    Hp = home[0].shape[-1]
    dz = np.zeros((R, NvS, Hp), dtype=np.uint16)
    dg = np.zeros((R, NvS, Hp), dtype=np.uint16)
    du = np.zeros((R, NvS, Hp), dtype=np.uint16)
    dx = np.zeros((R, NvS, H), dtype=np.uint16)
    rnd = lambda v: bf16_to_f32(f64_to_bf16(v)).astype(np.float64)
    for d in (range(R) if ranks is None else ranks):
        for row, lo, hi in _segments(plan, d):
            X = bf16_to_f32(x_nvs[d, lo:hi]).astype(np.float64)
            DY = bf16_to_f32(dy_nvs[d, lo:hi]).astype(np.float64)
            wg, wu, wd = (bf16_to_f32(resolve_row(plan, d, row, home[p], pool[p]))
                          .astype(np.float64) for p in range(3))
            outs = swiglu.backward(X, DY, wg, wu, wd, rnd=rnd)
            for tgt, v in zip((dz, dg, du, dx), outs):
                tgt[d, lo:hi] = f64_to_bf16(v)
    return dz, dg, du, dx


def expert_wgrad(plan, a_nvs, b_nvs, grad_home, reduce_buf):
    """dW_row += A_seg^T B_seg for every segment; rows below E go to
    grad_home, prefetch rows to the rank's reduce buffer.  Training only:
    needs B == E/R so that no row below E is written by a non-home rank."""
    if plan.B != plan.E // plan.R:
        raise ValueError("weight gradients need B == E/R")
    gh = grad_home.copy()
    rb = reduce_buf.copy()
    for d in range(plan.R):
        for row, lo, hi in _segments(plan, d):
            A = bf16_to_f32(a_nvs[d, lo:hi]).astype(np.float64)
            Bm = bf16_to_f32(b_nvs[d, lo:hi]).astype(np.float64)
            tgt = gh[row] if row < plan.E else rb[d, row - plan.E]
            tgt[...] = (tgt.astype(np.float64) + A.T @ Bm).astype(np.float32)
    return gh, rb


def reduce_grad(plan, grad_home, reduce_buf):
    """grad_home[e] += reduce_buf[d][j] for every used slot, d ascending, in
    fp32; then the used slots are zeroed for the next micro-batch."""
    gh = grad_home.copy()
    rb = reduce_buf.copy()
    for d in range(plan.R):
        for j in range(plan.B):
            e = plan.prefetch_src[d, j]
            if e >= 0:
                gh[e] = (gh[e] + rb[d, j]).astype(np.float32)
                rb[d, j] = 0.0
    return gh, rb
