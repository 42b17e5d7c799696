"""Python binding of libfa: exact IO-aware attention on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  The functions take torch
tensors for device memory and streams (torch is plumbing here) and keep the
C names:

* :func:`fa_fwd` -- O and LSE from Q, K, V
* :func:`fa_fwd_mxfp8` -- the same on fp8 codes with e8m0 block scales
* :func:`fa_fwd_bias`, :func:`fa_bwd_bias` -- forward and backward with an
  additive bias (and masks, as -inf) on the scaled scores
* :func:`fa_bwd` -- dQ, dK, dV from Q, K, V, O, dO, LSE (and a workspace)
* :func:`fa_bwd_noalloc` -- fa_bwd for callers that cannot allocate: delta in
  the library's per-GPU scratch instead of a workspace
* :func:`fa_bwd_delta`, :func:`fa_bwd_dkdv`, :func:`fa_bwd_dq` -- fa_bwd's stages,
  separately (for bf16 the dQ stage also writes delta)
* :func:`fa_std_fwd`, :func:`fa_std_workspace_size` -- standard attention with
  S and P written to device memory: the baseline of the IO comparison
* :func:`fa_bwd_workspace_size`, :func:`fa_status_string`
* :func:`fa_measure_mfma_rate` (module :mod:`.probe`, library libfa_probe.so,
  include/fa_probe.h) -- a measurement aid outside the attention library: the
  matrix-core rate on realistic operand bits, against which the kernels'
  rates are also read

There is no fallback: if a shared library is missing or fails to load, the
import of :mod:`exact_io_aware_11_amd._lib` (or :mod:`.probe`) raises.
"""
from __future__ import annotations

from ._lib import (FA_BF16, FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_FP32,
                   FA_FP8_E4M3, FA_NOALLOC_MAX_ROWS, FA_OK, FAError, lib)
from .api import (dtype_code, fa_bwd, fa_bwd_bias, fa_bwd_delta, fa_bwd_dkdv, fa_bwd_dq,
                  fa_bwd_noalloc,
                  fa_bwd_workspace_size, fa_fwd, fa_fwd_bias, fa_fwd_mxfp8,
                  fa_status_string, fa_std_fwd, fa_std_workspace_size, flops_bwd, flops_fwd)
from .probe import fa_measure_mfma_rate

__all__ = [
    "FA_FP32", "FA_BF16", "FA_FP8_E4M3", "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED",
    "FA_ERR_HIP", "FAError", "lib", "fa_fwd", "fa_fwd_bias", "fa_fwd_mxfp8", "fa_bwd",
    "fa_bwd_bias", "fa_bwd_delta", "fa_bwd_dkdv", "fa_measure_mfma_rate",
    "fa_bwd_dq", "fa_bwd_noalloc", "FA_NOALLOC_MAX_ROWS", "fa_bwd_workspace_size",
    "fa_std_fwd", "fa_std_workspace_size",
    "fa_status_string", "dtype_code", "flops_fwd", "flops_bwd",
]
