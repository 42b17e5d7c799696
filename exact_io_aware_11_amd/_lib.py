"""ctypes loader for libfa.so.  Raises at import time if the library is absent."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_FP32, FA_BF16, FA_FP8_E4M3 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_NOALLOC_MAX_ROWS = 1 << 22  # include/fa.h

# The entry points include/fa.h declares, with their ctypes signatures.
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_ll = ctypes.c_longlong
SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _f, _f, _f, _vp]),
    "fa_fwd_mxfp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]),
    "fa_bwd_workspace_size": (_sz, [_i, _i, _i, _i]),
    "fa_std_workspace_size": (_sz, [_i, _i, _i, _i]),
    "fa_std_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _f,
                    _i, _i, _vp]),
    "fa_fwd_bias": (_i, [_vp, _vp, _vp, _vp, _ll, _ll, _ll, _vp, _vp, _i, _i, _i, _i, _f, _i,
                         _i, _vp]),
    "fa_bwd_bias": (_i, [_vp, _vp, _vp, _vp, _ll, _ll, _ll, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _sz, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i,
                            _i, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
}
for _stage in ("fa_bwd_delta", "fa_bwd_dkdv", "fa_bwd_dq"):
    SIGNATURES[_stage] = SIGNATURES["fa_bwd"]


class FAError(RuntimeError):
    """A non-OK fa_status returned by the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status}")


def _check_loaded_torch() -> None:
    # torch must be loaded first: its HIP runtime carries the soname
    # libamdhip64.so.7 that libfa.so asks for, so both share ONE runtime (and
    # torch's streams and allocations are valid for our launches).  Loading
    # libfa.so first would pull in a second HIP runtime, and torch, which asks
    # for the unversioned name, would then load its own copy next to it.
    import torch  # noqa: F401


def _load() -> ctypes.CDLL:
    _check_loaded_torch()
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python exact_io_aware_11_amd/build.py` "
            "(there is no CPU fallback)")
    cdll = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(cdll, name)
        fn.restype = res
        fn.argtypes = args
    return cdll


lib = _load()
