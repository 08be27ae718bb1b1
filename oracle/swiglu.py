"""SwiGLU expert FFN, forward and backward, for one expert.  TEST
INFRASTRUCTURE ONLY.

MoonEP README (MoonshotAI/MoonEP mirror), "Usage > Integration": the expert
FFN applied to each segment is SwiGLU over the [H,H'] gate, up and down
projections.  The backward is not printed on any page (the framework owns the
expert FFN there); it follows from the forward by the chain rule:

  forward   G = X Wg,  U = X Wu,  Z = silu(G) * U,  Y = Z Wd^T
            silu(g) = g * sigma(g),  sigma(g) = 1 / (1 + exp(-g))
  backward  dZ = dY Wd
            dU = dZ * silu(G)
            dG = dZ * U * silu'(G),  silu'(g) = sigma(g) * (1 + g * (1 - sigma(g)))
            dX = dG Wg^T + dU Wu^T
  weights   dWg = X^T dG,  dWu = X^T dU,  dWd = dY^T Z

`rnd` is applied wherever a tensor is stored between two matrix products:
identity for the exact float64 functions (pinned by finite differences), bf16
round-to-nearest-even for the values the GPU path stores (Z, Y, dZ, dG, dU,
dX).  Products and sums are float64.
"""
import numpy as np


def _identity(v):
    return v


def sigma(g):
    return 1.0 / (1.0 + np.exp(-g))


def forward(x, wg, wu, wd, rnd=_identity):
    """x [n,H], wg/wu/wd [H,H'] float64 -> (z, y) float64 after `rnd`."""
    g = x @ wg
    u = x @ wu
    z = rnd(g * sigma(g) * u)
    y = rnd(z @ wd.T)
    return z, y


def backward(x, dy, wg, wu, wd, rnd=_identity):
    """x [n,H], dy [n,H] (gradient of the loss w.r.t. y), weights [H,H'] ->
    (dz, dg, du, dx), float64 after `rnd` at each stored tensor."""
    g = x @ wg
    u = x @ wu
    s = sigma(g)
    dz = rnd(dy @ wd)
    du = rnd(dz * (g * s))
    dg = rnd(dz * u * (s * (1.0 + g * (1.0 - s))))
    dx = rnd(dg @ wg.T + du @ wu.T)
    return dz, dg, du, dx
