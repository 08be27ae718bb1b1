"""Pins for the oracle's bf16 rounding: torch's float32 -> bfloat16
conversion (a library routine, round to nearest even) and hand-worked ties."""
import numpy as np
import torch

import oracle


def _torch_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_conversion_random():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32),
        (rng.standard_normal(10_000) * 1e30).astype(np.float32),
        (rng.standard_normal(10_000) * 1e-38).astype(np.float32),  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38], dtype=np.float32),
    ])
    assert (oracle.f32_to_bf16(x) == _torch_bits(x)).all()


def test_ties_round_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: the even neighbour is 1.0
    one = np.float32(1.0)
    half_ulp = np.float32(2.0 ** -8)
    x = np.array([one + half_ulp, one + 3 * half_ulp, np.float32(1.0 + 2.0 ** -8 + 2.0 ** -23)],
                 dtype=np.float32)
    got = oracle.bf16_to_f32(oracle.f32_to_bf16(x))
    assert got[0] == 1.0                       # tie -> even (mantissa 0)
    assert got[1] == np.float32(1.0 + 2.0 ** -6)  # tie -> even (mantissa 2)
    assert got[2] == np.float32(1.0 + 2.0 ** -7)  # above the tie -> up


def test_round_trip_exact_for_bf16_values():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(bits)
    ok = ~np.isnan(f)
    assert (oracle.f32_to_bf16(f[ok]) == bits[ok]).all()


def test_f64_path():
    x = np.array([1.0 + 2.0 ** -9, -2.5, 1e-3], dtype=np.float64)
    assert (oracle.f64_to_bf16(x) == _torch_bits(x.astype(np.float32))).all()
