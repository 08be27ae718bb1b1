"""Routing imbalance.  TEST INFRASTRUCTURE ONLY.

maxvio = max_e (T_e / T_bar) - 1, where T_e is the number of token-slots routed
to expert e and T_bar the count every expert would get under perfect balance
(MoonEP README, section "Performance"; MarkTechPost article, section "The
problem MoonEP targets").  T_e is summed over all R ranks, so
T_bar = R*S*K/E.  0 means perfectly balanced.
"""
import numpy as np


def expert_loads(topk: np.ndarray, E: int) -> np.ndarray:
    """T_e for e in [0,E): how many (r,s,k) pick expert e."""
    flat = np.asarray(topk).reshape(-1)
    T = np.zeros(E, dtype=np.int64)
    for e in flat.tolist():
        T[e] += 1
    return T


def maxvio(topk: np.ndarray, E: int) -> float:
    topk = np.asarray(topk)
    R, S, K = topk.shape
    T = expert_loads(topk, E).astype(np.float64)
    t_bar = R * S * K / E
    return float(T.max() / t_bar - 1.0)
