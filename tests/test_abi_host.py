"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moonep.h declares, sizes its buffers as the oracle
does, and rejects bad configurations and arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import moonep_synth as synth
import oracle
from grouped_gemm_moonep_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "moonep.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moonep_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = _abi.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = _abi.lib()
    assert lib.moonep_abi_version() == 1
    for s in range(7):
        assert _abi.status_string(s)
    assert _abi.status_string(99) == "unknown status"


def _cfg(w, **kw):
    d = dict(R=w.R, S=w.S, K=w.K, E=w.E, B=w.B, H=w.H, Hp=w.Hp,
             token_padding=w.token_padding, num_cus=0)
    d.update(kw)
    return _abi.config(**d)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_nvs_and_plan_sizes_match_oracle(name):
    w = synth.WORKLOADS[name]
    cfg = _cfg(w)
    NvS = oracle.nvs(w.S, w.K, w.E, w.R, w.token_padding)
    assert _abi.nvs(cfg) == NvS
    want = [w.R * w.E, w.R * w.S * w.K, w.R * NvS, w.R * (w.E + w.B), w.R * (w.E + w.B),
            w.R * w.B, 8 + 2 * w.R]
    got = [_abi.plan_len(cfg, i) for i in range(7)]
    assert got == want
    assert _abi.plan_len(cfg, 7) > 0
    assert _abi.plan_len(cfg, 8) == -1


BAD = [dict(E=6, R=4), dict(K=0), dict(K=9, E=8), dict(B=3), dict(B=-1), dict(S=0),
       dict(token_padding=0), dict(H=100), dict(Hp=32), dict(R=65, E=130), dict(E=2048, R=2),
       dict(num_cus=-1), dict(K=33, E=64),
       dict(H=32768, Hp=32768),                 # a weight row past 31-bit offsets
       dict(S=1 << 16, K=2, H=8192, Hp=64),     # a segment past 31-bit offsets
       dict(H=65536 + 64, Hp=64)]


@pytest.mark.parametrize("bad", BAD)
def test_bad_config_rejected_on_host(bad):
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    cfg = _cfg(w, **bad)
    lib = _abi.lib()
    assert lib.moonep_nvs(ctypes.byref(cfg)) == -1
    h = ctypes.c_void_p()
    assert lib.moonep_create(ctypes.byref(cfg), ctypes.byref(h)) == _abi.MOONEP_ERR_CONFIG
    assert not h.value


def test_null_arguments_rejected_on_host():
    lib = _abi.lib()
    plan = _abi.MoonepPlan()
    P3 = ctypes.c_void_p * 3
    ERR = _abi.MOONEP_ERR_ARG
    assert lib.moonep_create(None, None) == ERR
    assert lib.moonep_destroy(None) == _abi.MOONEP_OK
    assert lib.moonep_plan(None, None, None, ctypes.byref(plan), None) == ERR
    assert lib.moonep_dispatch(None, ctypes.byref(plan), None, 8, None, None, None, None) == ERR
    assert lib.moonep_combine(None, ctypes.byref(plan), None, 8, None, None, None, None) == ERR
    assert lib.moonep_copy_rows(None, ctypes.byref(plan), None, 8, None, None) == ERR
    assert lib.moonep_prefetch_weight(None, ctypes.byref(plan), P3(), P3(), None) == ERR
    assert lib.moonep_expert_ffn(None, ctypes.byref(plan), -1, None, P3(), P3(), None, None,
                                 None) == ERR
    assert lib.moonep_expert_gateup(None, ctypes.byref(plan), -1, None, P3(), P3(), None,
                                    None) == ERR
    assert lib.moonep_expert_down(None, ctypes.byref(plan), -1, None, P3(), P3(), None,
                                  None) == ERR
    assert lib.moonep_expert_ffn_bwd(None, ctypes.byref(plan), -1, None, None, P3(), P3(), None,
                                     None, None, None, None) == ERR
    assert lib.moonep_expert_wgrad(None, ctypes.byref(plan), -1, None, None, None, None,
                                   None) == ERR
    assert lib.moonep_reduce_grad(None, ctypes.byref(plan), P3(), P3(), None) == ERR
    assert lib.moonep_read_stats(None, ctypes.byref(plan), None, None) == ERR
    assert lib.moonep_vmm_granularity(None) == ERR
    out = ctypes.c_void_p()
    assert lib.moonep_symbuf_create(None, 2, None, ctypes.byref(out)) == ERR
    assert lib.moonep_symbuf_info(None, None) == ERR
    assert lib.moonep_symbuf_destroy(None) == _abi.MOONEP_OK
    assert lib.moonep_prefetch_weight_views(None, ctypes.byref(plan), P3(), None) == ERR
    assert lib.moonep_expert_ffn_views(None, ctypes.byref(plan), -1, None, P3(), None, None,
                                       None) == ERR
    assert lib.moonep_expert_ffn_bwd_views(None, ctypes.byref(plan), -1, None, None, P3(), None,
                                           None, None, None, None) == ERR


def test_noalloc_plan_checks_on_host():
    """moonep_plan_noalloc rejects, before touching a GPU: a bad configuration,
    missing or misaligned pointers, and a configuration whose planning
    scratch exceeds the library's fixed array (MOONEP_ERR_SCRATCH)."""
    lib = _abi.lib()
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    fake = ctypes.c_void_p(0x10000)          # never dereferenced on these paths
    full = _abi.MoonepPlan(*([0x10000] * len(_abi.PLAN_ARRAYS)))
    assert lib.moonep_plan_noalloc(ctypes.byref(_cfg(w, K=0)), fake, None, ctypes.byref(full),
                                   None) == _abi.MOONEP_ERR_CONFIG
    assert lib.moonep_plan_noalloc(None, fake, None, ctypes.byref(full),
                                   None) == _abi.MOONEP_ERR_CONFIG
    assert lib.moonep_plan_noalloc(ctypes.byref(_cfg(w)), None, None, ctypes.byref(full),
                                   None) == _abi.MOONEP_ERR_ARG
    assert lib.moonep_plan_noalloc(ctypes.byref(_cfg(w)), ctypes.c_void_p(0x10002), None,
                                   ctypes.byref(full), None) == _abi.MOONEP_ERR_ARG
    assert lib.moonep_plan_noalloc(ctypes.byref(_cfg(w)), fake, None,
                                   ctypes.byref(_abi.MoonepPlan()), None) == _abi.MOONEP_ERR_ARG
    # R * ceil(S/256) * E int32 of chunk counts alone: 8 * 782 * 256 > 2 MiB / 4
    big = _cfg(w, S=200_000, H=64, Hp=64)
    assert lib.moonep_nvs(ctypes.byref(big)) > 0
    assert lib.moonep_plan_noalloc(ctypes.byref(big), fake, None, ctypes.byref(full),
                                   None) == _abi.MOONEP_ERR_SCRATCH
    assert "scratch" in _abi.status_string(_abi.MOONEP_ERR_SCRATCH)


def test_dlpack_wrapper_layout():
    """The DLPack structures the binding builds by hand (to show library-owned
    device memory as torch tensors) import correctly; checked on host memory
    with device type CPU."""
    import numpy as np
    import torch
    a = np.arange(2 * 3 * 4, dtype=np.float32).reshape(2, 3, 4)
    t = _abi.wrap_memory(a.ctypes.data, (2, 3, 4), torch.float32, 1, 0)
    assert t.shape == (2, 3, 4) and t.dtype == torch.float32 and t.is_contiguous()
    assert t.data_ptr() == a.ctypes.data
    assert torch.equal(t, torch.from_numpy(a))
    t[1, 2, 3] = -5.0
    assert a[1, 2, 3] == -5.0
    src = torch.arange(16, dtype=torch.float32).to(torch.bfloat16)
    b = _abi.wrap_memory(src.data_ptr(), (4, 4), torch.bfloat16, 1, 0)
    assert b.dtype == torch.bfloat16 and torch.equal(b.reshape(-1), src)


GRIDS = [_abi.GRID_DISPATCH, _abi.GRID_COMBINE, _abi.GRID_COPY, _abi.GRID_PREFETCH,
         _abi.GRID_REDUCE_GRAD]


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_cu_budget_caps_every_data_movement_grid(name):
    """The launchers size their grids with the same host functions that
    moonep_launch_grid reports (README "API guide", num_sms): with a CU budget
    no data-movement launch exceeds num_cus * 8 workgroups, and the budget only
    ever lowers a grid; without one the grids cover every work item."""
    w = synth.WORKLOADS[name]
    for W in (8, 520, w.H, w.Hp):
        g0 = {k: _abi.launch_grid(_cfg(w), k, W) for k in GRIDS}
        assert all(v >= 1 for v in g0.values()), g0
        nvs = _abi.nvs(_cfg(w))
        # every (token, k, 1024-vector chunk) has a wave, padding items follow
        assert g0[_abi.GRID_DISPATCH] * 4 >= w.R * w.S * w.K * -(-(W // 8) // 1024)
        # every (token, 192-vector chunk) of combine, every slot row of copy
        assert g0[_abi.GRID_COMBINE] * 4 >= w.R * w.S * -(-(W // 8) // 192)
        assert g0[_abi.GRID_COPY] * 4 >= w.R * nvs
        assert g0[_abi.GRID_PREFETCH] % 3 == 0
        assert g0[_abi.GRID_REDUCE_GRAD] <= 256 * 8
        for num_cus in (1, 3, 32, 256):
            cap = num_cus * 8
            for k in GRIDS:
                g = _abi.launch_grid(_cfg(w, num_cus=num_cus), k, W)
                assert 1 <= g <= cap, (k, num_cus, g)
                want = min(g0[k], cap)
                if k == _abi.GRID_PREFETCH:
                    want = min(g0[k], cap // 3 * 3)
                assert g == want, (k, num_cus, g, g0[k])


def test_launch_grid_rejects_bad_arguments():
    w = synth.WORKLOADS["tiny_r4_s64_k2_e8"]
    c = _cfg(w)
    assert _abi.launch_grid(c, 99, 8) == -1
    for k in (_abi.GRID_DISPATCH, _abi.GRID_COMBINE, _abi.GRID_COPY):
        assert _abi.launch_grid(c, k, 0) == -1
        assert _abi.launch_grid(c, k, 12) == -1
    assert _abi.launch_grid(c, _abi.GRID_PREFETCH, 0) >= 3
    assert _abi.launch_grid(c, _abi.GRID_REDUCE_GRAD, 0, device_cus=0) == -1
    assert _abi.launch_grid(_cfg(w, K=0), _abi.GRID_DISPATCH, 8) == -1
