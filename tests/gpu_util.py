"""Helpers for the GPU parity tests: move seeded inputs to the device, read
results back, and build the oracle's expectation from the same inputs."""
import dataclasses

import numpy as np
import torch

import moonep_synth as synth
import oracle


def dev_bf16(a_u16):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def buffer_for(w, num_cus=0):
    from grouped_gemm_moonep_amd import Buffer
    return Buffer(R=w.R, S=w.S, K=w.K, E=w.E, B=w.B, H=w.H, Hp=w.Hp,
                  token_padding=w.token_padding, num_cus=num_cus)


def plan_host(buf, plan):
    torch.cuda.synchronize()
    R, S, K, E, B, NvS = buf.R, buf.S, buf.K, buf.E, buf.B, buf.NvS
    g = lambda n: plan.arrays[n].cpu().numpy()
    return dict(counts=g("counts").reshape(R, E), dest=g("dest").reshape(R, S, K),
                src=g("src").reshape(R, NvS), cu_seqlens=g("cu_seqlens").reshape(R, E + B),
                seg_tokens=g("seg_tokens").reshape(R, E + B),
                prefetch_src=g("prefetch_src").reshape(R, B), stats=g("stats"))


def workload(name, **kw):
    w = synth.WORKLOADS[name]
    return dataclasses.replace(w, **kw) if kw else w


def log(msg):
    print(f"[gpu] {msg}", flush=True)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def bf16_ulp(want_bits):
    """Spacing of bf16 values at |want| (one unit in the last place)."""
    w = np.asarray(want_bits, np.uint16)
    mag = oracle.bf16_to_f32(w & 0x7FFF).astype(np.float64)
    nxt = oracle.bf16_to_f32((w & 0x7FFF) + 1).astype(np.float64)
    return nxt - mag


def assert_close_bf16(got_bits, want_bits, rel=1e-2, abs_=2e-2, what="", ulps=1):
    """GEMM/FFN tolerance: rel-L2 <= 1e-2 and, element-wise,
    |got - want| <= max(2e-2, `ulps` bf16 ulps of want).  A bf16 output
    cannot be closer to an independently rounded reference than one ulp of its
    own grid, which exceeds 2e-2 once |want| >= 4; a value computed from
    another rounded bf16 intermediate (the FFN backward) may sit one more ulp
    away."""
    g = oracle.bf16_to_f32(got_bits).astype(np.float64)
    w = oracle.bf16_to_f32(want_bits).astype(np.float64)
    r = rel_l2(g, w)
    err = np.abs(g - w)
    bound = np.maximum(abs_, ulps * bf16_ulp(want_bits))
    m = float(err.max()) if g.size else 0.0
    worst = float((err / bound).max()) if g.size else 0.0
    # the plain element-wise figures, so that the ulp allowance cannot hide a
    # drift: how many elements exceed 2e-2 at all, and the mean signed error
    # against the reference's rms (a bias, which independent rounding keeps
    # near zero)
    n_over = int((err > abs_).sum())
    bias = float(np.mean(g - w) / max(np.sqrt(np.mean(w * w)), 1e-30)) if g.size else 0.0
    log(f"{what}: rel-L2 {r:.2e} max-abs {m:.2e} above {abs_:g}: {n_over}/{g.size} "
        f"bias/rms {bias:+.1e}")
    assert r <= rel and worst <= 1.0, \
        f"{what}: rel-L2 {r:.3e} max-abs {m:.3e} (worst err/bound {worst:.2f})"
    assert abs(bias) <= 1e-3, f"{what}: systematic error, mean/rms {bias:.3e}"
    return r, m
