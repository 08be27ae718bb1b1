"""CPU oracle for the MoonEP hot path.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never links, loads or calls it, and it
imports nothing from the GPU library or its Python binding.

Everything here is plain, slow, obviously-correct numpy / Python, written from
the pages' statement of the method:

* maxvio -- MoonEP README (MoonshotAI/MoonEP mirror), section "Performance";
  MarkTechPost article, section "The problem MoonEP targets".
* the S x K invariant and redundant-expert planning -- README items 1-2 and
  "How to set B"; the planner's exact steps are not printed on any page, so
  the spec the oracle follows (P1-P9 in planner.py) is this project's reading.
* dispatch / combine / prefetch / reduce_grad -- README "API guide".
* the grouped SwiGLU FFN over one [E+B,H,H'] tensor per projection addressed
  by cu_seqlens -- README "Usage > Integration > Weight buffer"; its backward
  (swiglu.py) follows from the forward by the chain rule and is pinned by
  finite differences.

Floating point: hidden states, weights and expert outputs are bf16 and route
weights and gradients fp32, as the README's API guide fixes; matrix products
are taken in float64 and rounded to bf16 where the stored tensor is bf16.
Combine and reduce_grad are defined in fp32 with a fixed summation order so
that the GPU result is comparable bit for bit.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: torch's bf16 conversion, closed forms for balanced and adversarial
routing, hand-worked plans, brute-force optima, a dense per-token MoE written
independently of the planner, and dense per-expert gradients.
"""
from .bf16 import bf16_to_f32, f32_to_bf16, f64_to_bf16
from .maxvio import expert_loads, maxvio
from .planner import Plan, nvs, plan
from .moe import (combine, combine_rows, dispatch, expert_ffn, expert_ffn_backward,
                  prefetch_weight, reduce_grad, expert_wgrad, resolve_row)
from .dense import dense_moe, dense_expert_grad, ffn_token, ffn_token_backward
from . import swiglu
from .bruteforce import min_duplicates

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "f64_to_bf16", "expert_loads", "maxvio",
    "Plan", "nvs", "plan", "dispatch", "combine", "combine_rows", "prefetch_weight",
    "expert_ffn_backward", "ffn_token_backward", "swiglu",
    "expert_ffn", "expert_wgrad", "reduce_grad", "resolve_row", "dense_moe",
    "dense_expert_grad", "ffn_token", "min_duplicates",
]
