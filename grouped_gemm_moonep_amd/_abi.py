"""ctypes binding of libmoonep.so (the C ABI declared in include/moonep.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; shapes, dtypes, devices and contiguity are checked here
because the C ABI receives bare pointers.  Every computation happens in the
library's gfx950 kernels; if the library cannot be loaded, importing fails.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoonep.so")

(MOONEP_OK, MOONEP_ERR_ARG, MOONEP_ERR_CONFIG, MOONEP_ERR_MODE, MOONEP_ERR_HIP, MOONEP_ERR_NOMEM,
 MOONEP_ERR_SCRATCH) = range(7)
STAT_ERROR, STAT_DUPS, STAT_MAX_LOAD, STAT_DONATIONS, STAT_PAD_ROWS, STAT_MAXVIO = range(6)
STAT_FIXED = 8
PLAN_ARRAYS = ["counts", "dest", "src", "cu_seqlens", "seg_tokens", "prefetch_src", "stats", "aux"]


class MoonepConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("R", "S", "K", "E", "B", "H", "Hp", "token_padding", "num_cus")]


class MoonepPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PLAN_ARRAYS]


class MoonepSymbufInfo(ctypes.Structure):
    _fields_ = [("views", ctypes.c_void_p), ("home", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("row_bytes", ctypes.c_int64), ("physical_bytes", ctypes.c_int64),
                ("granularity", ctypes.c_int64)]


class MoonepError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib():
    """Load libmoonep.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python grouped_gemm_moonep_amd/build.py`")
    try:
        import torch  # noqa: F401  (share torch's HIP runtime if it is loaded)
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P3 = ctypes.c_void_p * 3
    sig = {
        "moonep_abi_version": (i32, []),
        "moonep_status_string": (ctypes.c_char_p, [i32]),
        "moonep_nvs": (i64, [ctypes.POINTER(MoonepConfig)]),
        "moonep_plan_len": (i64, [ctypes.POINTER(MoonepConfig), i32]),
        "moonep_launch_grid": (i64, [ctypes.POINTER(MoonepConfig), i32, i32, i32]),
        "moonep_create": (i32, [ctypes.POINTER(MoonepConfig), ctypes.POINTER(vp)]),
        "moonep_destroy": (i32, [vp]),
        "moonep_plan": (i32, [vp, vp, vp, ctypes.POINTER(MoonepPlan), vp]),
        "moonep_plan_noalloc": (i32, [ctypes.POINTER(MoonepConfig), vp, vp,
                                      ctypes.POINTER(MoonepPlan), vp]),
        "moonep_dispatch": (i32, [vp, ctypes.POINTER(MoonepPlan), vp, i32, vp, vp, vp, vp]),
        "moonep_combine": (i32, [vp, ctypes.POINTER(MoonepPlan), vp, i32, vp, vp, vp, vp]),
        "moonep_copy_rows": (i32, [vp, ctypes.POINTER(MoonepPlan), vp, i32, vp, vp]),
        "moonep_prefetch_weight": (i32, [vp, ctypes.POINTER(MoonepPlan), P3, P3, vp]),
        "moonep_expert_ffn": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, P3, P3, vp, vp, vp]),
        "moonep_expert_gateup": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, P3, P3, vp, vp]),
        "moonep_expert_down": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, P3, P3, vp, vp]),
        "moonep_expert_ffn_bwd": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, vp, P3, P3, vp,
                                        vp, vp, vp, vp]),
        "moonep_expert_wgrad": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, vp, vp, vp, vp]),
        "moonep_reduce_grad": (i32, [vp, ctypes.POINTER(MoonepPlan), P3, P3, vp]),
        "moonep_read_stats": (i32, [vp, ctypes.POINTER(MoonepPlan), vp, vp]),
        "moonep_vmm_granularity": (i32, [ctypes.POINTER(i64)]),
        "moonep_symbuf_create": (i32, [vp, i32, vp, ctypes.POINTER(vp)]),
        "moonep_symbuf_info": (i32, [vp, ctypes.POINTER(MoonepSymbufInfo)]),
        "moonep_symbuf_destroy": (i32, [vp]),
        "moonep_prefetch_weight_views": (i32, [vp, ctypes.POINTER(MoonepPlan), P3, vp]),
        "moonep_expert_ffn_views": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, P3, vp, vp,
                                          vp]),
        "moonep_expert_ffn_bwd_views": (i32, [vp, ctypes.POINTER(MoonepPlan), i32, vp, vp, P3,
                                              vp, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    if L.moonep_abi_version() != 1:
        raise ImportError("libmoonep.so ABI version mismatch")
    _lib = L
    return L


def status_string(s):
    return lib().moonep_status_string(int(s)).decode()


def check(status, where):
    if status != MOONEP_OK:
        raise MoonepError(status, where)


def config(R, S, K, E, B, H, Hp, token_padding, num_cus=0):
    return MoonepConfig(R, S, K, E, B, H, Hp, token_padding, num_cus)


def nvs(cfg: MoonepConfig) -> int:
    return int(lib().moonep_nvs(ctypes.byref(cfg)))


def plan_len(cfg: MoonepConfig, which: int) -> int:
    return int(lib().moonep_plan_len(ctypes.byref(cfg), which))


GRID_DISPATCH, GRID_COMBINE, GRID_COPY, GRID_PREFETCH, GRID_REDUCE_GRAD = range(5)


def launch_grid(cfg: MoonepConfig, which: int, W: int = 0, device_cus: int = 256) -> int:
    """Workgroups a data-movement call would launch (host only)."""
    return int(lib().moonep_launch_grid(ctypes.byref(cfg), which, W, device_cus))


def ptr3(ts):
    return (ctypes.c_void_p * 3)(*[None if t is None else t.data_ptr() for t in ts])


# -- device memory the library owns, seen as torch tensors (DLPack) ----------
# DLPack's C structures (dlpack.h, version 0.x "DLManagedTensor"), declared
# here because the capsule is built with ctypes.

class _DLDevice(ctypes.Structure):
    _fields_ = [("device_type", ctypes.c_int32), ("device_id", ctypes.c_int32)]


class _DLDataType(ctypes.Structure):
    _fields_ = [("code", ctypes.c_uint8), ("bits", ctypes.c_uint8), ("lanes", ctypes.c_uint16)]


class _DLTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("device", _DLDevice), ("ndim", ctypes.c_int32),
                ("dtype", _DLDataType), ("shape", ctypes.POINTER(ctypes.c_int64)),
                ("strides", ctypes.POINTER(ctypes.c_int64)), ("byte_offset", ctypes.c_uint64)]


class _DLManagedTensor(ctypes.Structure):
    _fields_ = [("dl_tensor", _DLTensor), ("manager_ctx", ctypes.c_void_p),
                ("deleter", ctypes.c_void_p)]


_DL_ROCM = 10
_DL_FLOAT, _DL_BFLOAT = 2, 4
# The consumer reads the managed tensor again when its tensor dies (to find the
# deleter, which is NULL here), so the structures stay alive for the process.
_dl_keep = []


def device_tensor(ptr, shape, dtype, device_index):
    """Torch tensor over `ptr` (device memory owned by the library, not by
    torch): dense row-major `shape` of bf16 or fp32.  The tensor does not
    keep the memory alive; its owner must outlive every use of it."""
    return wrap_memory(ptr, shape, dtype, _DL_ROCM, device_index)


def wrap_memory(ptr, shape, dtype, device_type, device_index):
    """DLPack import of foreign memory (device_type 10 = ROCm, 1 = CPU)."""
    import torch
    code, bits = {torch.bfloat16: (_DL_BFLOAT, 16), torch.float32: (_DL_FLOAT, 32)}[dtype]
    shp = (ctypes.c_int64 * len(shape))(*shape)
    mt = _DLManagedTensor()
    mt.dl_tensor.data = ptr
    mt.dl_tensor.device = _DLDevice(device_type, device_index)
    mt.dl_tensor.ndim = len(shape)
    mt.dl_tensor.dtype = _DLDataType(code, bits, 1)
    mt.dl_tensor.shape = shp
    mt.dl_tensor.strides = None
    mt.dl_tensor.byte_offset = 0
    mt.manager_ctx = None
    mt.deleter = None
    _dl_keep.append((mt, shp))
    new_capsule = ctypes.pythonapi.PyCapsule_New
    new_capsule.restype = ctypes.py_object
    new_capsule.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_void_p]
    cap = new_capsule(ctypes.addressof(mt), b"dltensor", None)
    return torch.utils.dlpack.from_dlpack(cap)
