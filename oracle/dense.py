"""Dense, unbalanced per-token MoE reference.  TEST INFRASTRUCTURE ONLY.

No planner, no slots, no prefetch: every token is run through each of its K
experts with that expert's home weights and the K outputs are summed with the
route weights.  This is what combine(FFN(dispatch(x))) must equal whatever the
plan (MoonEP README item 1 and "API guide": the balanced path only moves
tokens and weights around, it changes no result).

Arithmetic per expert output: G = x Wg, U = x Wu (float64), Z rounded to
bf16, Y = Z Wd^T rounded to bf16; the sum over k uses fp32 products and fp32
adds in ascending k, as the combine reading states.
"""
import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16, f64_to_bf16
from . import swiglu


def _rnd_bf16(v):
    """float64 -> nearest bf16 value (round to nearest even), as float64."""
    return bf16_to_f32(f64_to_bf16(v)).astype(np.float64)


def ffn_token(x_bits, wg_bits, wu_bits, wd_bits):
    """One token (or a batch [n,H]) through one expert: returns (z, y) bits."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    wg = bf16_to_f32(wg_bits).astype(np.float64)
    wu = bf16_to_f32(wu_bits).astype(np.float64)
    wd = bf16_to_f32(wd_bits).astype(np.float64)
    g = x @ wg
    u = x @ wu
    z = f64_to_bf16(g / (1.0 + np.exp(-g)) * u)
    y = f64_to_bf16(bf16_to_f32(z).astype(np.float64) @ wd.T)
    return z, y


def ffn_token_backward(x_bits, dy_bits, wg_bits, wu_bits, wd_bits):
    """Backward of one expert's SwiGLU for a batch of tokens [n,H] given the
    gradient dy [n,H] of its output: returns (dz, dg, du, dx) bf16 bits, each
    rounded where it is stored (see swiglu.backward)."""
    f = lambda b: bf16_to_f32(b).astype(np.float64)
    out = swiglu.backward(f(x_bits), f(dy_bits), f(wg_bits), f(wu_bits), f(wd_bits),
                          rnd=_rnd_bf16)
    return tuple(f64_to_bf16(v) for v in out)


def dense_moe(topk, rw, x, home):
    """topk [R,S,K], rw [R,S,K] f32, x [R,S,H] bits, home = (gate, up, down)
    [E,H,H'] bits -> out [R,S,H] bits."""
    R, S, K = topk.shape
    H = x.shape[-1]
    tokens = x.reshape(R * S, H)
    ids = topk.reshape(R * S, K)
    ys = np.zeros((R * S, K, H), dtype=np.uint16)
    for e in np.unique(ids):
        t, k = np.nonzero(ids == e)
        _, y = ffn_token(tokens[t], home[0][e], home[1][e], home[2][e])
        ys[t, k] = y
    w = rw.reshape(R * S, K).astype(np.float32)
    acc = None
    for k in range(K):
        pk = (w[:, k:k + 1] * bf16_to_f32(ys[:, k])).astype(np.float32)
        acc = pk if acc is None else (acc + pk).astype(np.float32)
    return f32_to_bf16(acc).reshape(R, S, H)


def dense_expert_grad(topk, a, b, E):
    """Unbalanced per-expert weight gradient in float64:
    dW_e = sum over tokens routed to e of a_token (outer) b_token,
    a [R,S,H] bits, b [R,S,H'] bits -> [E,H,H'] float64."""
    R, S, K = topk.shape
    A = bf16_to_f32(a.reshape(R * S, -1)).astype(np.float64)
    Bm = bf16_to_f32(b.reshape(R * S, -1)).astype(np.float64)
    ids = topk.reshape(R * S, K)
    out = np.zeros((E, A.shape[1], Bm.shape[1]), dtype=np.float64)
    for e in range(E):
        t = np.nonzero((ids == e).any(axis=1))[0]
        if t.size:
            out[e] = A[t].T @ Bm[t]
    return out
