"""ctypes view of libdash.so (the C ABI declared in include/dash.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# DASH_LIB names another build of the same library (the CPU ABI tests use it for
# the host-sanitized build); the default is the in-tree libdash.so.
LIB_PATH = os.environ.get("DASH_LIB") or os.path.join(PKG, "libdash.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dash.h")

DASH_F32 = 0
DASH_BF16 = 1

STATUS = {0: "DASH_OK", 1: "DASH_ERR_INVALID_ARG", 2: "DASH_ERR_UNSUPPORTED", 3: "DASH_ERR_WORKSPACE", 4: "DASH_ERR_HIP"}


class DashParams(ctypes.Structure):
    """Mirror of ``dash_params`` (passed by value)."""

    _fields_ = [
        ("chunk_size", ctypes.c_int),
        ("alpha", ctypes.c_float),
        ("n_iter", ctypes.c_int),
        ("scaling_factor", ctypes.c_float),
        ("causal", ctypes.c_int),
        ("estimate_diagonal", ctypes.c_int),
    ]


class DashError(RuntimeError):
    def __init__(self, where: str, status: int):
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "dash_default_params": (None, [ctypes.POINTER(DashParams)]),
    "dash_status_string": (ctypes.c_char_p, [_I]),
    "dash_summarize": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _I, _I, DashParams, _P]),
    "dash_summarize_backward": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, DashParams, _P, _P, _P, _P]),
    "dash_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, DashParams]),
    "dash_prefill_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, DashParams, ctypes.c_longlong]),
    "dash_prefill_counters": (_I, [_P, _SZ, _I, _I, _I, _I, _I, DashParams, _P, _P]),
    "dash_route": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, DashParams, _P, _P, _I, _P, _SZ, _P]),
    "dash_sparse_attn_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, DashParams, _P, _P, _SZ, _P]),
    "dash_sparse_attn_decode": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _I, _I, DashParams, _P, _P, _SZ, _P]),
    "dash_decode_step_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _I, _I, DashParams, _P, _P, _P,
                                      _I, _P]),
    "dash_decode_noalloc_max_bytes": (_SZ, []),
    "dash_sparse_attn_prefill_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                               DashParams, _P, _P, _P, _P, _P, _SZ, _P]),
    "dash_backward_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, DashParams]),
    "entmax_attn": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _F, _I, _I, _P, _P, _P, _P]),
    "entmax_attn_backward": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _F, _I, _P, _P, _P, _P, _P]),
    "entmax_rows": (_I, [_P, _P, _I, _I, _I, _F, _I, _P, _P]),
    "entmax_rows_backward": (_I, [_P, _P, _P, _I, _I, _I, _F, _P]),
}

_lib = None


def header_symbols() -> list:
    """Function names declared in include/dash.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_]+)\s*\(", text, flags=re.M)))


def load() -> ctypes.CDLL:
    """Load libdash.so once and attach the argument types of every entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m adaptive_sparse_long_amd.build` "
            "(the HIP library is the only implementation)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def params(chunk_size=64, alpha=1.5, n_iter=10, scaling_factor=1.0, causal=True, estimate_diagonal=True) -> DashParams:
    return DashParams(int(chunk_size), float(alpha), int(n_iter), float(scaling_factor), int(bool(causal)), int(bool(estimate_diagonal)))


def check(status: int, where: str) -> None:
    if status != 0:
        raise DashError(where, status)
