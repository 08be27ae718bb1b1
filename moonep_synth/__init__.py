"""Seeded synthetic inputs for the MoonEP hot path.

This module only *draws* inputs: workload shapes, router outputs (top-K expert
ids and route weights), hidden states, expert weights and output gradients.
It holds none of the method's arithmetic (no planning, no maxvio, no buffer
sizing, no rounding code of its own: float -> bf16 goes through torch's
conversion).  Both the CPU oracle and the GPU path are fed from here, so the
two sides always see identical tensors.

Workloads follow the problem statement of the MoonEP README (MoonshotAI/MoonEP
mirror), section "Usage > Integration": S tokens per rank, top-K routing over
E experts spread over R EP ranks, B prefetch slots per rank, hidden size H,
expert intermediate size H'.  The benchmark set-up of the MarkTechPost article
(k7ail translation, section "Benchmarks against DeepEP v2") drives routing from
a shared seed at a range of imbalance targets; here that becomes:

* logits ~ N(0,1), shape [R,S,E] float32, from sub-stream (seed, 1);
* a Zipf-like popularity bias  bias_e = -s * ln(e+1)  (expert 0 hottest);
* top-K of logits+bias with ties to the lower expert id, k ordered by
  descending score;
* route weights = softmax over the K chosen biased scores (float32).

The bias strength s for a target imbalance is read from a table that a
committed script (tests/golden/make_zipf_scales.py) fits with the oracle.
Exactly balanced and adversarial routings have closed forms (below).
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_REPO = os.path.dirname(_HERE)
ZIPF_TABLE = os.path.join(_REPO, "tests", "golden", "zipf_scales.json")

# sub-stream ids of np.random.default_rng([seed, k])
STREAM_HIDDEN, STREAM_LOGITS, STREAM_PERM, STREAM_DY = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload: R ranks x S tokens, top-K of E experts, B prefetch slots."""
    name: str
    R: int
    S: int
    K: int
    E: int
    B: int
    H: int
    Hp: int
    token_padding: int

    def as_dict(self):
        return dataclasses.asdict(self)


WORKLOADS = {
    w.name: w
    for w in [
        # small case: the oracle finishes every stage in well under a second
        Workload("tiny_r4_s64_k2_e8", R=4, S=64, K=2, E=8, B=2, H=128, Hp=256,
                 token_padding=16),
        # mid-size forward, also the shape of the training-backward case
        Workload("mid_r8_s1024_k4_e32", R=8, S=1024, K=4, E=32, B=4, H=1024,
                 Hp=2048, token_padding=128),
        # headline forward: the README's own Buffer example (S=4096, H=7168,
        # K=8, E=256, 8 ranks, token_padding=128) with B = E/R
        Workload("fwd_r8_s4096_k8_e256", R=8, S=4096, K=8, E=256, B=32,
                 H=7168, Hp=2048, token_padding=128),
        # inference prefetch mode, B < E/R (README "How to set B": 3-4)
        Workload("infer_r8_s128_k8_e256_b4", R=8, S=128, K=8, E=256, B=4,
                 H=7168, Hp=2048, token_padding=128),
        # the shape of the pages' own benchmark (README "Performance"): EP 8,
        # S=8192, E=384, K=8, H=7168, H'=2048; training prefetch B = E/R
        Workload("pages_r8_s8192_k8_e384", R=8, S=8192, K=8, E=384, B=48,
                 H=7168, Hp=2048, token_padding=128),
    ]
}
# the training backward runs on the mid-size shapes
WORKLOADS["bwd_r8_s1024_k4_e32"] = dataclasses.replace(
    WORKLOADS["mid_r8_s1024_k4_e32"], name="bwd_r8_s1024_k4_e32")

# imbalance targets swept per workload ("adv" = every token on experts 0..K-1)
SWEEPS = {
    "tiny_r4_s64_k2_e8": [1.0],
    "pages_r8_s8192_k8_e384": [0.2, 1.0, 10.0, 20.0],
    "mid_r8_s1024_k4_e32": [0.0, 0.5, 1.0, 2.0],
    "fwd_r8_s4096_k8_e256": [0.0, 0.5, 1.0, 2.0, 4.0, "adv"],
    "infer_r8_s128_k8_e256_b4": [1.0, 4.0],
    "bwd_r8_s1024_k4_e32": [0.0, 2.0],
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


# ----------------------------------------------------------------- routing
def _softmax_f32(scores: np.ndarray) -> np.ndarray:
    z = scores.astype(np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=-1, keepdims=True)).astype(np.float32)


def routing_zipf(w: Workload, s: float, seed: int = 0):
    """Top-K routing with a Zipf popularity bias of strength s.

    Returns (topk [R,S,K] int32, rw [R,S,K] float32)."""
    logits = rng(seed, STREAM_LOGITS).standard_normal(
        (w.R, w.S, w.E), dtype=np.float32)
    bias = (-s * np.log(np.arange(1, w.E + 1, dtype=np.float64))).astype(np.float32)
    scores = logits + bias
    # stable sort of the negated score: equal scores keep ascending expert id
    order = np.argsort(-scores, axis=-1, kind="stable")[..., : w.K]
    chosen = np.take_along_axis(scores, order, axis=-1)
    return order.astype(np.int32), _softmax_f32(chosen)


def routing_balanced(w: Workload, seed: int = 0):
    """Exactly balanced routing: slot (r,s,k) -> pi(((r*S+s)*K+k) mod E) for a
    seeded permutation pi.  K consecutive residues are distinct, so every token
    has K distinct experts, and every expert gets R*S*K/E slots."""
    assert (w.R * w.S * w.K) % w.E == 0 and w.K <= w.E
    perm = rng(seed, STREAM_PERM).permutation(w.E).astype(np.int32)
    idx = np.arange(w.R * w.S * w.K, dtype=np.int64).reshape(w.R, w.S, w.K)
    topk = perm[idx % w.E]
    logits = rng(seed, STREAM_LOGITS).standard_normal((w.R, w.S, w.K), dtype=np.float32)
    logits = -np.sort(-logits, axis=-1)          # k in descending score order
    return topk.astype(np.int32), _softmax_f32(logits)


def routing_adversarial(w: Workload, seed: int = 0):
    """Every token picks experts 0..K-1 (slot k -> expert k)."""
    topk = np.broadcast_to(np.arange(w.K, dtype=np.int32), (w.R, w.S, w.K)).copy()
    logits = rng(seed, STREAM_LOGITS).standard_normal((w.R, w.S, w.K), dtype=np.float32)
    logits = -np.sort(-logits, axis=-1)
    return topk, _softmax_f32(logits)


def _topk_of(scores: np.ndarray, K: int):
    order = np.argsort(-scores, axis=-1, kind="stable")[..., :K]
    chosen = np.take_along_axis(scores, order, axis=-1)
    return order.astype(np.int32), _softmax_f32(chosen)


def routing_rank_skew(w: Workload, strength: float, seed: int = 0):
    """Every rank prefers the experts homed on the next rank: logits ~ N(0,1)
    plus `strength` on experts of group (r+1) mod R for the tokens of rank r
    (the home groups' loads stay equal while every rank sends its traffic away)."""
    logits = rng(seed, STREAM_LOGITS).standard_normal((w.R, w.S, w.E), dtype=np.float32)
    L = w.E // w.R
    for r in range(w.R):
        g = (r + 1) % w.R
        logits[r, :, g * L:(g + 1) * L] += np.float32(strength)
    return _topk_of(logits, w.K)


def routing_hot(w: Workload, nhot: int, seed: int = 0):
    """Experts 0..nhot-1 (nhot <= K) in every token, the rest of its K at random."""
    logits = rng(seed, STREAM_LOGITS).standard_normal((w.R, w.S, w.E), dtype=np.float32)
    logits[..., :nhot] += np.float32(100.0)
    return _topk_of(logits, w.K)


def zipf_scale(name: str, target) -> float:
    with open(ZIPF_TABLE) as f:
        table = json.load(f)
    return float(table[name][str(float(target))])


def routing(w: Workload, target, seed: int = 0):
    """Routing at a sweep point: 0.0 -> balanced, "adv" -> adversarial,
    otherwise Zipf with the fitted strength for that imbalance target."""
    if target == "adv":
        return routing_adversarial(w, seed)
    if float(target) == 0.0:
        return routing_balanced(w, seed)
    return routing_zipf(w, zipf_scale(w.name, target), seed)


# ------------------------------------------------------------ dense tensors
def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) through torch's own conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def hidden(w: Workload, seed: int = 0, width=None) -> np.ndarray:
    """Token-major hidden states [R,S,W] as bf16 bits, N(0,1)."""
    W = w.H if width is None else width
    x = rng(seed, STREAM_HIDDEN).standard_normal((w.R, w.S, W), dtype=np.float32)
    return to_bf16_bits(x)


def grad_out(w: Workload, width: int, seed: int = 0, stream_offset: int = 0) -> np.ndarray:
    """Token-major output gradient [R,S,width] as bf16 bits, N(0,1)."""
    g = rng(seed, STREAM_DY + 16 * stream_offset).standard_normal(
        (w.R, w.S, width), dtype=np.float32)
    return to_bf16_bits(g)


def expert_weights_host(w: Workload, proj: int, seed: int = 0, rows=None) -> np.ndarray:
    """Home expert weights of one projection (0 gate, 1 up, 2 down) as bf16
    bits [len(rows), H, H'], N(0, 0.02); row e has its own generator
    (seed, 10+proj, e) so any subset of rows can be drawn on its own."""
    rows = range(w.E) if rows is None else rows
    out = np.empty((len(rows), w.H, w.Hp), dtype=np.uint16)
    for i, e in enumerate(rows):
        v = np.random.default_rng([seed, 10 + proj, int(e)]).standard_normal(
            (w.H, w.Hp), dtype=np.float32) * np.float32(0.02)
        out[i] = to_bf16_bits(v)
    return out


def expert_weights_device(w: Workload, proj: int, out, seed: int = 0):
    """Fill a [E,H,H'] bfloat16 CUDA tensor with N(0,0.02) drawn on the GPU,
    one seeded torch generator per expert row (for sizes where drawing on the
    host would take minutes).  The oracle copies back only the rows it uses."""
    import torch
    assert out.shape == (w.E, w.H, w.Hp) and out.dtype == torch.bfloat16
    g = torch.Generator(device=out.device)
    tmp = torch.empty((w.H, w.Hp), dtype=torch.float32, device=out.device)
    for e in range(w.E):
        g.manual_seed((seed * 1_000_003 + (10 + proj)) * 1_000_003 + e)
        tmp.normal_(0.0, 0.02, generator=g)
        out[e].copy_(tmp)
    return out
