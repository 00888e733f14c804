"""ctypes binding of libsdtw.so: the C ABI of include/sdtw.h, same names.

Argument marshalling only -- every step of the computation runs in the HIP
kernels behind these calls.  Pointers are passed as integers (device
addresses), streams as integers (hipStream_t handles, 0 = null stream).
If the library is not built this module raises at first use; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdtw.so")
STRESS_LIB_PATH = os.path.join(HERE, "libsdtw_stress.so")   # debug build, tests only

SDTW_OK = 0
SDTW_ERR_INVALID_ARG = 1
SDTW_ERR_WORKSPACE = 2
SDTW_ERR_HIP = 3
SDTW_ERR_UNSUPPORTED = 4
SDTW_ERR_STALLED = 5

SDTW_MODE_UNFUSED = 0
SDTW_MODE_FUSED = 1
SDTW_MODE_INFERENCE = 2
SDTW_MODE_CHECKPOINT = 3
SDTW_MODE_UNFUSED_LOWMEM = 4

# (name, restype, argtypes) for every entry point declared in include/sdtw.h.
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_F = ctypes.c_float
_I = ctypes.c_int
SIGNATURES = {
    "sdtw_abi_version": (_I, []),
    "sdtw_status_string": (ctypes.c_char_p, [_I]),
    "sdtw_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I]),
    "sdtw_dist": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "sdtw_forward": (_I, [_P, _P, _I64, _I64, _I64, _I64, _F, _I, _P,
                          ctypes.c_size_t, _P, _P]),
    "sdtw_backward": (_I, [_P, _P, _I64, _I64, _I64, _I64, _F, _I, _P,
                           ctypes.c_size_t, _P, _P, _P, _P, _P]),
    "sdtw_workspace_status": (_I, [_P, ctypes.c_size_t, _I64, _I64, _I64, _I64, _I, _P]),
    "sdtw_debug_wait_limit": (_I, [_I64]),
    "sdtw_forward_static": (_I, [_P, _P, _I64, _I64, _I64, _I64, _F, _P, _P]),
    "sdtw_timing": (_I, [_I]),
    "sdtw_timing_collect": (_I, [ctypes.POINTER(ctypes.c_char_p),
                                 ctypes.POINTER(ctypes.c_float), _I]),
}

_lib = None


class SdtwError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sdtw_status_string(status)} (status {status})")


def load(path: str) -> ctypes.CDLL:
    """A build of the library at `path` with every entry point's signature
    set (lib() for libsdtw.so; the stress tests also load the stress build)."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m "
            "differentiable_series_alignment_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def sdtw_abi_version() -> int:
    return lib().sdtw_abi_version()


def sdtw_status_string(status: int) -> str:
    return lib().sdtw_status_string(int(status)).decode()


def sdtw_workspace_bytes(B: int, N: int, M: int, D: int, mode: int) -> int:
    return int(lib().sdtw_workspace_bytes(B, N, M, D, mode))


def sdtw_dist(x: int, y: int, dist: int, B: int, N: int, M: int, D: int,
              stream: int = 0) -> int:
    return lib().sdtw_dist(x, y, dist, B, N, M, D, stream)


def sdtw_forward(x: int, y: int, B: int, N: int, M: int, D: int, gamma: float,
                 mode: int, workspace: int, workspace_bytes: int, loss: int,
                 stream: int = 0) -> int:
    return lib().sdtw_forward(x, y, B, N, M, D, gamma, mode, workspace,
                              workspace_bytes, loss, stream)


def sdtw_backward(x: int, y: int, B: int, N: int, M: int, D: int, gamma: float,
                  mode: int, workspace: int, workspace_bytes: int, grad_loss: int,
                  grad_x: int | None, grad_y: int | None, align: int | None,
                  stream: int = 0) -> int:
    return lib().sdtw_backward(x, y, B, N, M, D, gamma, mode, workspace,
                               workspace_bytes, grad_loss, grad_x, grad_y, align,
                               stream)


def sdtw_workspace_status(workspace: int, workspace_bytes: int, B: int, N: int, M: int,
                          D: int, mode: int, stream: int = 0) -> int:
    return lib().sdtw_workspace_status(workspace, workspace_bytes, B, N, M, D, mode, stream)


def sdtw_debug_wait_limit(polls: int) -> int:
    return lib().sdtw_debug_wait_limit(int(polls))


SDTW_STATIC_SCRATCH_BYTES = 16 << 20


def sdtw_forward_static(x: int, y: int, B: int, N: int, M: int, D: int, gamma: float,
                        loss: int, stream: int = 0) -> int:
    return lib().sdtw_forward_static(x, y, B, N, M, D, gamma, loss, stream)


def sdtw_timing(on: bool) -> int:
    return lib().sdtw_timing(1 if on else 0)


def sdtw_timing_collect(cap: int = 4096) -> list[tuple[str, float]]:
    """(kernel name, milliseconds) of the launches recorded since the last
    collect, in launch order.  The record list is process-wide: a collect
    drains the launches of every host thread and stream."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = lib().sdtw_timing_collect(names, ms, cap)
    if n < 0:
        raise SdtwError(-n, "sdtw_timing_collect")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


def check(status: int, where: str) -> None:
    if status != SDTW_OK:
        raise SdtwError(status, where)
