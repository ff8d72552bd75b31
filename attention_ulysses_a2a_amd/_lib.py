"""ctypes loader for libxstage.so (built in-tree by ``attention_ulysses_a2a_amd.build``).

There is no fallback: if the library is missing, every entry point raises
``LibraryMissing``.  The library is never rebuilt implicitly here.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxstage.so")

XSTAGE_MAX_P = 64
XSTAGE_OK = 0
XSTAGE_ERR_INVALID = 1
XSTAGE_ERR_UNSUPPORTED = 2
XSTAGE_ERR_HIP = 3


class LibraryMissing(RuntimeError):
    pass


class XStageError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_name(status)} ({status})")


class MoeParams(ctypes.Structure):
    """Mirror of xstage_moe_params_t."""

    _fields_ = [
        ("E", ctypes.c_int),
        ("d_model", ctypes.c_int),
        ("d_ff", ctypes.c_int),
        ("experts_per_wave", ctypes.c_int),
        ("schedule", ctypes.c_int),
        ("expert_offsets", ctypes.POINTER(ctypes.c_int)),
        ("x", ctypes.c_void_p),
        ("w1", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("h", ctypes.c_void_p),
        ("dst_slab", ctypes.c_void_p),
        ("dst_row", ctypes.c_void_p),
        ("P", ctypes.c_int),
        ("out", ctypes.POINTER(ctypes.c_void_p)),
        ("out_rows", ctypes.POINTER(ctypes.c_int)),
        ("stamps", ctypes.c_void_p),
    ]


class BGParams(ctypes.Structure):
    """Mirror of xstage_bg_params_t."""

    _fields_ = [
        ("K", ctypes.c_int),
        ("rounds", ctypes.c_int),
        ("n_dst_sets", ctypes.c_int),
        ("nontemporal", ctypes.c_int),
        ("V_bytes", ctypes.c_ulonglong),
        ("gap_fma_iters", ctypes.c_uint),
        ("dst", ctypes.c_void_p),
        ("stamps", ctypes.c_void_p),
        ("sync", ctypes.c_void_p),
        ("sync_timeout_ticks", ctypes.c_ulonglong),
    ]


_vp = ctypes.c_void_p
_i = ctypes.c_int
_PP = ctypes.POINTER(ctypes.c_void_p)

_u64 = ctypes.c_ulonglong
_f = ctypes.c_float
_WS = [_vp, _u64]  # split_ws, split_ws_bytes

SIGNATURES = {
    "xstage_attn_a2a_fwd": (_i, [_vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_attn_split_ws_size": (_i, [_i, _i, _i, _i, ctypes.POINTER(_u64)]),
    "xstage_attn_a2a_fwd_noalloc": (_i, [_vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _f, _vp]),
    "xstage_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_a2a_scatter": (_i, [_vp, _PP, _i, _i, _i, _i, _i, _vp]),
    "xstage_attn_a2a_unfused": (_i, [_vp, _vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_attn_a2a_fwd_strided": (_i, [_vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_ulysses_attn_fwd": (_i, [_PP, _PP, _PP, _PP, _i, _i, _i, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_ulysses_gather": (_i, [_PP, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "xstage_a2a_scatter_strided": (_i, [_vp, _PP, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "xstage_ulysses_attn_unfused": (_i, [_PP, _PP, _PP, _vp, _PP, _i, _i, _i, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_ulysses_attn_fwd_kv_staged": (
        _i, [_PP, _PP, _PP, _vp, _PP, _i, _i, _i, _i, _i, _i, _i, _f] + _WS + [_vp]),
    "xstage_attn_a2a_plan": (_i, [_i, _i, _i, _i, _u64, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "xstage_attn_a2a_wg_rows": (_i, [_i, _i, _i, _i, _u64, ctypes.POINTER(_i)]),
    "xstage_attn_a2a_schedule": (_i, [_i, _i, _i, _i, _u64, _i] + [ctypes.POINTER(_i)] * 5),
    "xstage_attn_a2a_fwd_traced": (_i, [_vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _f, _i, _vp] + _WS + [_vp]),
    "xstage_attn_a2a_fwd_paced": (_i, [_vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "xstage_attn_a2a_fwd_nsplit": (_i, [_vp, _vp, _vp, _PP, _i, _i, _i, _i, _i, _f, _i] + _WS + [_vp]),
    "xstage_attn_nsplit_ws_size": (_i, [_i, _i, _i, _i, _i, ctypes.POINTER(_u64)]),
    "xstage_attn_a2a_paced_plan": (_i, [_i, _i, _i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "xstage_moe_waves_run": (_i, [ctypes.POINTER(MoeParams), _vp]),
    "xstage_moe_waves_plan": (_i, [_i, ctypes.POINTER(_i), _i, _i, _i, _i] + [ctypes.POINTER(_i)] * 4),
    "xstage_burst_gap_run": (_i, [ctypes.POINTER(BGParams), _vp]),
    "xstage_wallclock_hz": (_i, [ctypes.POINTER(ctypes.c_double)]),
    "xstage_bg_t_iss": (ctypes.c_double, [ctypes.c_double] * 4),
    "xstage_bg_pacing_chunks": (_i, [ctypes.c_double] * 6 + [_i, ctypes.POINTER(ctypes.c_double)]),
    "xstage_status_str": (ctypes.c_char_p, [_i]),
}

# split_ws_bytes value asking the plan queries for the unconstrained (full-speed) plan
WS_FULL = (1 << 64) - 1

_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} not found: build it with `python -m attention_ulysses_a2a_amd.build` "
                "(there is no CPU or PyTorch fallback)"
            )
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_name(status: int) -> str:
    try:
        return lib().xstage_status_str(int(status)).decode()
    except LibraryMissing:
        return {0: "XSTAGE_OK", 1: "XSTAGE_ERR_INVALID", 2: "XSTAGE_ERR_UNSUPPORTED", 3: "XSTAGE_ERR_HIP"}.get(
            int(status), "XSTAGE_UNKNOWN_STATUS")


def ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[ctypes.c_void_p(int(p)) if p else None for p in ptrs])
    return ctypes.cast(arr, _PP), arr
