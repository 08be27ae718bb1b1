"""MoonEP hot path on AMD MI355X (gfx950): Python binding of libmoonep.so.

`Buffer` mirrors the MoonEP README's Buffer (MoonshotAI/MoonEP mirror,
"API guide"), for all R EP ranks of one GPU at once.  Each method is one call
of the C ABI of the same name (include/moonep.h) with torch tensors supplying
device memory and the current stream; nothing is computed in Python.

    buf = Buffer(R=8, S=4096, K=8, E=256, B=32, H=7168, Hp=2048, token_padding=128)
    plan = buf.plan(topk)                           # moonep_plan
    x_nvs, rw_nvs = buf.dispatch(plan, x, rw)       # moonep_dispatch
    buf.prefetch_weight(plan, home, pool)           # moonep_prefetch_weight
    buf.expert_ffn(plan, x_nvs, home, pool, z, y)   # moonep_expert_ffn
                                                    # (= expert_gateup + expert_down)
    out, rw_sk = buf.combine(plan, y, rw_nvs)       # moonep_combine

`SymmetricBuffer` is the README's [E+B,H,H'] weight (or fp32 gradient) buffer
of one projection on virtual memory (moonep_symbuf_*): per-rank views whose
rows [0,E) map every rank's home chunk, with the *_views methods addressing
experts purely by row index.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import MoonepError, lib  # noqa: F401

__all__ = ["Buffer", "Plan", "SymmetricBuffer", "MoonepError", "lib", "vmm_granularity"]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_ptr(t, dtype, shape, name, nullable=False):
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class Plan:
    """Device arrays of one plan (see moonep_plan_t)."""

    def __init__(self, cfg, device):
        self.arrays = {}
        self._store = []
        for i, name in enumerate(_abi.PLAN_ARRAYS):
            n = _abi.plan_len(cfg, i)
            # zero-length arrays (B = 0) still get a valid device pointer
            store = torch.empty(max(n, 1), dtype=torch.int32, device=device)
            self.arrays[name] = store[:n]
            self._store.append(store)
        self.struct = _abi.MoonepPlan(*[s.data_ptr() for s in self._store])

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays")
        if arrays is not None and name in arrays:
            return arrays[name]
        raise AttributeError(name)


class Buffer:
    """Handle of the MoonEP path for R ranks on the current device."""

    def __init__(self, R, S, K, E, B=None, H=7168, Hp=2048, token_padding=128, num_cus=0,
                 device="cuda"):
        if B is None:
            B = E // R
        self.R, self.S, self.K, self.E, self.B = R, S, K, E, B
        self.H, self.Hp, self.token_padding = H, Hp, token_padding
        self.device = torch.device(device)
        self.cfg = _abi.config(R, S, K, E, B, H, Hp, token_padding, num_cus)
        self.NvS = _abi.nvs(self.cfg)
        if self.NvS < 0:
            raise MoonepError(_abi.MOONEP_ERR_CONFIG, "Buffer")
        self._h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _abi.check(lib().moonep_create(ctypes.byref(self.cfg), ctypes.byref(self._h)),
                       "moonep_create")

    # -- lifecycle -----------------------------------------------------------
    def destroy(self):
        if self._h:
            _abi.check(lib().moonep_destroy(self._h), "moonep_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def new_plan(self):
        return Plan(self.cfg, self.device)

    # -- calls -----------------------------------------------------------------
    def plan(self, topk, tokens_per_expert=None, plan=None):
        plan = plan or self.new_plan()
        R, S, K, E = self.R, self.S, self.K, self.E
        p_topk = _dev_ptr(topk, torch.int32, (R, S, K), "topk")
        p_tpe = _dev_ptr(tokens_per_expert, torch.int32, (R, E), "tokens_per_expert", True)
        _abi.check(lib().moonep_plan(self._h, p_topk, p_tpe, ctypes.byref(plan.struct), _stream()),
                   "moonep_plan")
        return plan

    def plan_noalloc(self, topk, tokens_per_expert=None, plan=None):
        """moonep_plan_noalloc: the same plan as `plan`, computed without the
        handle's scratch and without allocating device memory (the library's
        fixed per-GPU scratch array; concurrent calls on one GPU race).  Only
        `plan=None` allocates here, in Python, for the plan arrays."""
        plan = plan or self.new_plan()
        R, S, K, E = self.R, self.S, self.K, self.E
        p_topk = _dev_ptr(topk, torch.int32, (R, S, K), "topk")
        p_tpe = _dev_ptr(tokens_per_expert, torch.int32, (R, E), "tokens_per_expert", True)
        _abi.check(lib().moonep_plan_noalloc(ctypes.byref(self.cfg), p_topk, p_tpe,
                                             ctypes.byref(plan.struct), _stream()),
                   "moonep_plan_noalloc")
        return plan

    def copy_rows(self, plan, src_nvs, dst_nvs=None):
        """The used slots of every rank from src_nvs to dst_nvs (moonep_copy_rows)."""
        R, NvS = self.R, self.NvS
        W = src_nvs.shape[-1]
        if dst_nvs is None:
            dst_nvs = torch.empty_like(src_nvs)
        args = (_dev_ptr(src_nvs, torch.bfloat16, (R, NvS, W), "src_nvs"), int(W),
                _dev_ptr(dst_nvs, torch.bfloat16, (R, NvS, W), "dst_nvs"))
        _abi.check(lib().moonep_copy_rows(self._h, ctypes.byref(plan.struct), *args, _stream()),
                   "moonep_copy_rows")
        return dst_nvs

    def _comm(self, W, device):
        """The communication buffer of the copy mode (zero_copy=False), one per
        row width, owned by this Buffer."""
        bufs = self.__dict__.setdefault("_comm_bufs", {})
        if W not in bufs:
            bufs[W] = torch.empty((self.R, self.NvS, W), dtype=torch.bfloat16, device=device)
        return bufs[W]

    def dispatch(self, plan, x, rw=None, x_nvs=None, rw_nvs=None, zero_copy=True):
        """zero_copy=False (the README's copy mode): dispatch into this Buffer's
        communication buffer, then copy the used slots into x_nvs."""
        if not zero_copy:
            comm, rw_nvs = self.dispatch(plan, x, rw, x_nvs=self._comm(x.shape[-1], x.device),
                                         rw_nvs=rw_nvs)
            return self.copy_rows(plan, comm, x_nvs), rw_nvs
        R, S, K, NvS = self.R, self.S, self.K, self.NvS
        W = x.shape[-1]
        if x_nvs is None:
            x_nvs = torch.empty((R, NvS, W), dtype=torch.bfloat16, device=x.device)
        if rw is not None and rw_nvs is None:
            rw_nvs = torch.empty((R, NvS), dtype=torch.float32, device=x.device)
        args = (_dev_ptr(x, torch.bfloat16, (R, S, W), "x"), int(W),
                _dev_ptr(rw, torch.float32, (R, S, K), "rw", True),
                _dev_ptr(x_nvs, torch.bfloat16, (R, NvS, W), "x_nvs"),
                _dev_ptr(rw_nvs, torch.float32, (R, NvS), "rw_nvs", True))
        _abi.check(lib().moonep_dispatch(self._h, ctypes.byref(plan.struct), *args, _stream()),
                   "moonep_dispatch")
        return x_nvs, rw_nvs

    def combine(self, plan, y_nvs, rw_nvs=None, out=None, rw_sk=None, gather_rw=True,
                zero_copy=True):
        """zero_copy=False (the README's copy mode): copy the used slots of
        y_nvs into this Buffer's communication buffer first, then combine."""
        if not zero_copy:
            comm = self.copy_rows(plan, y_nvs, self._comm(y_nvs.shape[-1], y_nvs.device))
            return self.combine(plan, comm, rw_nvs, out, rw_sk, gather_rw)
        R, S, K, NvS = self.R, self.S, self.K, self.NvS
        W = y_nvs.shape[-1]
        if out is None:
            out = torch.empty((R, S, W), dtype=torch.bfloat16, device=y_nvs.device)
        if rw_nvs is not None and rw_sk is None and gather_rw:
            rw_sk = torch.empty((R, S, K), dtype=torch.float32, device=y_nvs.device)
        args = (_dev_ptr(y_nvs, torch.bfloat16, (R, NvS, W), "y_nvs"), int(W),
                _dev_ptr(rw_nvs, torch.float32, (R, NvS), "rw_nvs", True),
                _dev_ptr(out, torch.bfloat16, (R, S, W), "out"),
                _dev_ptr(rw_sk, torch.float32, (R, S, K), "rw_sk", True))
        _abi.check(lib().moonep_combine(self._h, ctypes.byref(plan.struct), *args, _stream()),
                   "moonep_combine")
        return out, rw_sk

    def _weights(self, ts, pool, used=(0, 1, 2)):
        R, E, B, H, Hp = self.R, self.E, self.B, self.H, self.Hp
        if len(ts) != 3:
            raise ValueError("three projections (gate, up, down) expected")
        shape = (R, B, H, Hp) if pool else (E, H, Hp)
        for i, t in enumerate(ts):
            if t is None and (i not in used or (pool and B == 0)):
                continue
            _dev_ptr(t, torch.bfloat16, shape, f"{'pool' if pool else 'home'}[{i}]")
        return _abi.ptr3(ts)

    def prefetch_weight(self, plan, home, pool):
        _abi.check(lib().moonep_prefetch_weight(self._h, ctypes.byref(plan.struct),
                                                self._weights(home, False),
                                                self._weights(pool, True), _stream()),
                   "moonep_prefetch_weight")

    def expert_ffn(self, plan, x_nvs, home, pool, z_ws=None, y_nvs=None, rank=-1):
        R, NvS, H, Hp = self.R, self.NvS, self.H, self.Hp
        if z_ws is None:
            z_ws = torch.empty((R, NvS, Hp), dtype=torch.bfloat16, device=x_nvs.device)
        if y_nvs is None:
            y_nvs = torch.empty((R, NvS, H), dtype=torch.bfloat16, device=x_nvs.device)
        args = (int(rank), _dev_ptr(x_nvs, torch.bfloat16, (R, NvS, H), "x_nvs"),
                self._weights(home, False), self._weights(pool, True),
                _dev_ptr(z_ws, torch.bfloat16, (R, NvS, Hp), "z_ws"),
                _dev_ptr(y_nvs, torch.bfloat16, (R, NvS, H), "y_nvs"))
        _abi.check(lib().moonep_expert_ffn(self._h, ctypes.byref(plan.struct), *args, _stream()),
                   "moonep_expert_ffn")
        return z_ws, y_nvs

    def _views(self, views):
        R, E, B, H, Hp = self.R, self.E, self.B, self.H, self.Hp
        if len(views) != 3:
            raise ValueError("three projections (gate, up, down) expected")
        for i, t in enumerate(views):
            _dev_ptr(t, torch.bfloat16, (R, E + B, H, Hp), f"views[{i}]")
        return _abi.ptr3(views)

    def prefetch_weight_views(self, plan, views):
        """prefetch_weight over per-rank [E+B] views (views[p] [R,E+B,H,Hp])."""
        _abi.check(lib().moonep_prefetch_weight_views(self._h, ctypes.byref(plan.struct),
                                                      self._views(views), _stream()),
                   "moonep_prefetch_weight_views")

    def expert_ffn_views(self, plan, x_nvs, views, z_ws=None, y_nvs=None, rank=-1):
        """expert_ffn with experts located by row index in rank d's [E+B] view."""
        R, NvS, H, Hp = self.R, self.NvS, self.H, self.Hp
        if z_ws is None:
            z_ws = torch.empty((R, NvS, Hp), dtype=torch.bfloat16, device=x_nvs.device)
        if y_nvs is None:
            y_nvs = torch.empty((R, NvS, H), dtype=torch.bfloat16, device=x_nvs.device)
        args = (int(rank), _dev_ptr(x_nvs, torch.bfloat16, (R, NvS, H), "x_nvs"),
                self._views(views),
                _dev_ptr(z_ws, torch.bfloat16, (R, NvS, Hp), "z_ws"),
                _dev_ptr(y_nvs, torch.bfloat16, (R, NvS, H), "y_nvs"))
        _abi.check(lib().moonep_expert_ffn_views(self._h, ctypes.byref(plan.struct), *args,
                                                 _stream()), "moonep_expert_ffn_views")
        return z_ws, y_nvs

    def expert_gateup(self, plan, x_nvs, home, pool, z_nvs=None, rank=-1):
        R, NvS, H, Hp = self.R, self.NvS, self.H, self.Hp
        if z_nvs is None:
            z_nvs = torch.empty((R, NvS, Hp), dtype=torch.bfloat16, device=x_nvs.device)
        args = (int(rank), _dev_ptr(x_nvs, torch.bfloat16, (R, NvS, H), "x_nvs"),
                self._weights(home, False, (0, 1)), self._weights(pool, True, (0, 1)),
                _dev_ptr(z_nvs, torch.bfloat16, (R, NvS, Hp), "z_nvs"))
        _abi.check(lib().moonep_expert_gateup(self._h, ctypes.byref(plan.struct), *args,
                                              _stream()), "moonep_expert_gateup")
        return z_nvs

    def expert_down(self, plan, z_nvs, home, pool, y_nvs=None, rank=-1):
        R, NvS, H, Hp = self.R, self.NvS, self.H, self.Hp
        if y_nvs is None:
            y_nvs = torch.empty((R, NvS, H), dtype=torch.bfloat16, device=z_nvs.device)
        args = (int(rank), _dev_ptr(z_nvs, torch.bfloat16, (R, NvS, Hp), "z_nvs"),
                self._weights(home, False, (2,)), self._weights(pool, True, (2,)),
                _dev_ptr(y_nvs, torch.bfloat16, (R, NvS, H), "y_nvs"))
        _abi.check(lib().moonep_expert_down(self._h, ctypes.byref(plan.struct), *args,
                                            _stream()), "moonep_expert_down")
        return y_nvs

    def expert_ffn_bwd(self, plan, x_nvs, dy_nvs, home, pool, dz_ws=None, dg_nvs=None,
                       du_nvs=None, dx_nvs=None, rank=-1):
        """Backward of the grouped SwiGLU FFN: returns (dz_ws, dg_nvs, du_nvs,
        dx_nvs); dx_nvs may be dy_nvs or x_nvs (in place)."""
        R, NvS, H, Hp = self.R, self.NvS, self.H, self.Hp
        dev = x_nvs.device
        new = lambda W: torch.empty((R, NvS, W), dtype=torch.bfloat16, device=dev)
        dz_ws = new(Hp) if dz_ws is None else dz_ws
        dg_nvs = new(Hp) if dg_nvs is None else dg_nvs
        du_nvs = new(Hp) if du_nvs is None else du_nvs
        dx_nvs = new(H) if dx_nvs is None else dx_nvs
        args = (int(rank), _dev_ptr(x_nvs, torch.bfloat16, (R, NvS, H), "x_nvs"),
                _dev_ptr(dy_nvs, torch.bfloat16, (R, NvS, H), "dy_nvs"),
                self._weights(home, False), self._weights(pool, True),
                _dev_ptr(dz_ws, torch.bfloat16, (R, NvS, Hp), "dz_ws"),
                _dev_ptr(dg_nvs, torch.bfloat16, (R, NvS, Hp), "dg_nvs"),
                _dev_ptr(du_nvs, torch.bfloat16, (R, NvS, Hp), "du_nvs"),
                _dev_ptr(dx_nvs, torch.bfloat16, (R, NvS, H), "dx_nvs"))
        _abi.check(lib().moonep_expert_ffn_bwd(self._h, ctypes.byref(plan.struct), *args,
                                               _stream()), "moonep_expert_ffn_bwd")
        return dz_ws, dg_nvs, du_nvs, dx_nvs

    def expert_ffn_bwd_views(self, plan, x_nvs, dy_nvs, views, dz_ws=None, dg_nvs=None,
                             du_nvs=None, dx_nvs=None, rank=-1):
        """expert_ffn_bwd with experts located by row index in rank d's [E+B] view."""
        R, NvS, H, Hp = self.R, self.NvS, self.H, self.Hp
        dev = x_nvs.device
        new = lambda W: torch.empty((R, NvS, W), dtype=torch.bfloat16, device=dev)
        dz_ws = new(Hp) if dz_ws is None else dz_ws
        dg_nvs = new(Hp) if dg_nvs is None else dg_nvs
        du_nvs = new(Hp) if du_nvs is None else du_nvs
        dx_nvs = new(H) if dx_nvs is None else dx_nvs
        args = (int(rank), _dev_ptr(x_nvs, torch.bfloat16, (R, NvS, H), "x_nvs"),
                _dev_ptr(dy_nvs, torch.bfloat16, (R, NvS, H), "dy_nvs"),
                self._views(views),
                _dev_ptr(dz_ws, torch.bfloat16, (R, NvS, Hp), "dz_ws"),
                _dev_ptr(dg_nvs, torch.bfloat16, (R, NvS, Hp), "dg_nvs"),
                _dev_ptr(du_nvs, torch.bfloat16, (R, NvS, Hp), "du_nvs"),
                _dev_ptr(dx_nvs, torch.bfloat16, (R, NvS, H), "dx_nvs"))
        _abi.check(lib().moonep_expert_ffn_bwd_views(self._h, ctypes.byref(plan.struct), *args,
                                                     _stream()), "moonep_expert_ffn_bwd_views")
        return dz_ws, dg_nvs, du_nvs, dx_nvs

    def expert_wgrad(self, plan, a_nvs, b_nvs, grad_home, reduce_buf, rank=-1):
        R, NvS, E, B, H, Hp = self.R, self.NvS, self.E, self.B, self.H, self.Hp
        args = (int(rank), _dev_ptr(a_nvs, torch.bfloat16, (R, NvS, H), "a_nvs"),
                _dev_ptr(b_nvs, torch.bfloat16, (R, NvS, Hp), "b_nvs"),
                _dev_ptr(grad_home, torch.float32, (E, H, Hp), "grad_home"),
                _dev_ptr(reduce_buf, torch.float32, (R, B, H, Hp), "reduce_buf"))
        _abi.check(lib().moonep_expert_wgrad(self._h, ctypes.byref(plan.struct), *args, _stream()),
                   "moonep_expert_wgrad")

    def reduce_grad(self, plan, grad_home, reduce_buf):
        R, E, B, H, Hp = self.R, self.E, self.B, self.H, self.Hp
        for i in range(3):
            _dev_ptr(grad_home[i], torch.float32, (E, H, Hp), f"grad_home[{i}]")
            _dev_ptr(reduce_buf[i], torch.float32, (R, B, H, Hp), f"reduce_buf[{i}]")
        _abi.check(lib().moonep_reduce_grad(self._h, ctypes.byref(plan.struct),
                                            _abi.ptr3(grad_home), _abi.ptr3(reduce_buf),
                                            _stream()),
                   "moonep_reduce_grad")

    def read_stats(self, plan):
        import numpy as np
        out = np.zeros(_abi.STAT_FIXED + 2 * self.R, dtype=np.int32)
        _abi.check(lib().moonep_read_stats(self._h, ctypes.byref(plan.struct),
                                           out.ctypes.data_as(ctypes.c_void_p), _stream()),
                   "moonep_read_stats")
        return out


def vmm_granularity():
    """Minimum virtual-memory allocation granularity of the current device, bytes."""
    g = ctypes.c_int64()
    _abi.check(lib().moonep_vmm_granularity(ctypes.byref(g)), "moonep_vmm_granularity")
    return int(g.value)


class SymmetricBuffer:
    """One projection's [E+B,H,H'] buffer for the R ranks of `buf`, built on
    virtual memory by the library (moonep_symbuf_create): bf16 weights (README
    "Weight buffer") or fp32 gradients ("Gradient buffer").

    views [R,E+B,H,Hp]: rank d's contiguous [E+B] range; rows [0,E) map the R
                        home chunks, rows [E,E+B) rank d's own slot chunk
    home  [E,H,Hp]:     the home chunks (home[p] / grad_home of the other calls)
    slots [R,B,H,Hp]:   the slot chunks (pool[p] / the [R,B] reduce view)

    The three tensors alias the same physical memory.  They do not own it:
    drop them before destroy().  `slots_from`: another SymmetricBuffer whose
    slot chunks this one maps (one prefetch pool shared by every layer)."""

    def __init__(self, buf, dtype=torch.bfloat16, slots_from=None):
        elem = {torch.bfloat16: 2, torch.float32: 4}.get(dtype)
        if elem is None:
            raise TypeError("SymmetricBuffer holds bf16 weights or fp32 gradients")
        self._b = ctypes.c_void_p()
        dev = buf.device if buf.device.index is not None else \
            torch.device("cuda", torch.cuda.current_device())
        share = slots_from._b if slots_from is not None else None
        with torch.cuda.device(dev):
            _abi.check(lib().moonep_symbuf_create(buf._h, elem, share, ctypes.byref(self._b)),
                       "moonep_symbuf_create")
        info = _abi.MoonepSymbufInfo()
        _abi.check(lib().moonep_symbuf_info(self._b, ctypes.byref(info)), "moonep_symbuf_info")
        self.row_bytes = int(info.row_bytes)
        self.physical_bytes = int(info.physical_bytes)
        self.granularity = int(info.granularity)
        R, E, B, H, Hp = buf.R, buf.E, buf.B, buf.H, buf.Hp
        self.views = _abi.device_tensor(info.views, (R, E + B, H, Hp), dtype, dev.index)
        self.home = _abi.device_tensor(info.home, (E, H, Hp), dtype, dev.index)
        self.slots = (_abi.device_tensor(info.slots, (R, B, H, Hp), dtype, dev.index) if B
                      else torch.empty((R, 0, H, Hp), dtype=dtype, device=dev))

    def destroy(self):
        if self._b:
            self.views = self.home = self.slots = None
            _abi.check(lib().moonep_symbuf_destroy(self._b), "moonep_symbuf_destroy")
            self._b = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# fail at import time, loudly, when the native library is missing
lib()
