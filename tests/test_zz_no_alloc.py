"""moonep_plan_noalloc (the allocation-free planning entry point, its scratch
in the library's fixed per-GPU array) against moonep_plan (the handle's
allocated scratch), through the C ABI: every plan array bit-identical, on
calls in a row whose sizes shrink and grow again (the array keeps the last
call's contents), with and without tokens_per_expert, and the plan also
matching the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from grouped_gemm_moonep_amd import _abi
from gpu_util import buffer_for, dev, log

pytestmark = pytest.mark.gpu

FILL = -1234567


def _fresh_plan(buf):
    p = buf.new_plan()
    for t in p._store:
        t.fill_(FILL)
    return p


def _noalloc(buf, topk, tpe, plan):
    st = _abi.lib().moonep_plan_noalloc(
        ctypes.byref(buf.cfg), ctypes.c_void_p(topk.data_ptr()),
        None if tpe is None else ctypes.c_void_p(tpe.data_ptr()),
        ctypes.byref(plan.struct), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _abi.check(st, "moonep_plan_noalloc")


@pytest.mark.parametrize("seq", [
    # larger, then smaller, then the larger again
    [("mid_r8_s1024_k4_e32", 2.0, False), ("tiny_r4_s64_k2_e8", 1.0, True),
     ("mid_r8_s1024_k4_e32", "adv", True)],
    [("fwd_r8_s4096_k8_e256", 4.0, False), ("mid_r8_s1024_k4_e32", 0.0, False)],
])
def test_noalloc_plan_equals_handle_plan(seq):
    for name, target, with_tpe in seq:
        w = synth.WORKLOADS[name]
        log(f"plan_noalloc {name} target={target} tpe={with_tpe}")
        topk, _ = synth.routing(w, target)
        t = dev(topk)
        tpe = (dev(oracle.plan(topk, w.E, w.B, w.token_padding).counts.astype(np.int32))
               if with_tpe else None)
        buf = buffer_for(w)
        want = _fresh_plan(buf)
        buf.plan(t, tpe, plan=want)
        got = _fresh_plan(buf)
        _noalloc(buf, t, tpe, got)
        torch.cuda.synchronize()
        for n in _abi.PLAN_ARRAYS:
            assert torch.equal(got.arrays[n], want.arrays[n]), f"{name} {target}: {n}"
        assert int(got.stats[0]) == 0
        p = oracle.plan(topk, w.E, w.B, w.token_padding)
        cu = got.cu_seqlens.cpu().numpy().reshape(w.R, w.E + w.B)
        assert np.array_equal(cu, p.cu_seqlens)
        assert np.array_equal(got.dest.cpu().numpy().reshape(w.R, w.S, w.K), p.dest)
        buf.destroy()


def test_noalloc_plan_binding_and_bad_routing():
    """The binding's plan_noalloc is the same call; an out-of-range expert id
    sets the sticky error flag exactly as moonep_plan does."""
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    topk, _ = synth.routing(w, 1.0)
    bad = topk.copy()
    bad[1, 3, 0] = w.E + 5
    buf = buffer_for(w)
    for tk in (topk, bad):
        want = _fresh_plan(buf)
        buf.plan(dev(tk), plan=want)
        got = _fresh_plan(buf)
        buf.plan_noalloc(dev(tk), plan=got)
        torch.cuda.synchronize()
        for n in _abi.PLAN_ARRAYS:
            assert torch.equal(got.arrays[n], want.arrays[n]), n
    assert int(got.stats[0]) == 1          # MOONEP_ROUTE_ID_RANGE
    buf.destroy()
