"""ctypes binding of libfa_probe.so (include/fa_probe.h): the matrix-core rate
probe, a measurement aid kept out of the attention library.  Raises at import
time if the library is absent (no fallback)."""
from __future__ import annotations

import ctypes
import os

from ._lib import FA_BF16, FA_FP8_E4M3, FA_OK, FAError, _check_loaded_torch

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_probe.so")
# the entry points include/fa_probe.h declares, with their ctypes signatures
SIGNATURES = {"fa_measure_mfma_rate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_int, ctypes.c_void_p])}


def _load() -> ctypes.CDLL:
    _check_loaded_torch()
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                          "`python exact_io_aware_11_amd/build.py`")
    cdll = ctypes.CDLL(PROBE_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(cdll, name)
        fn.restype = res
        fn.argtypes = args
    return cdll


probe_lib = _load()


def fa_measure_mfma_rate(out, blocks: int, iters: int, fp8: bool = False, stream=None):
    """Enqueue the matrix-core rate probe (include/fa_probe.h); out is a float32
    device tensor of at least blocks * 512 elements.  Returns the FLOPs the
    launch performs."""
    import torch

    from .api import _check_device, _stream_handle

    _check_device("out", out)
    if out.dtype != torch.float32 or out.numel() < blocks * 512:
        raise ValueError("out must be float32 with blocks * 512 elements")
    st = probe_lib.fa_measure_mfma_rate(out.data_ptr(), int(blocks), int(iters),
                                        FA_FP8_E4M3 if fp8 else FA_BF16, _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, f"fa_measure_mfma_rate: status {st}")
    return float(blocks) * 8 * iters * 8 * (131072 if fp8 else 32768)
