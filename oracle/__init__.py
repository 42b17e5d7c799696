"""Double-precision CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The HIP library
and its Python binding never import it, and it never imports them.

The arithmetic lives in ``fa_oracle.c`` (plain C, double precision, pthreads
over heads and row chunks).  This module builds that file with gcc on first
use (or through :func:`build`) and wraps it with ctypes and numpy.

What each function computes, and the passage it follows (pages: "FlashAttention-1:
eliminating IO", deep-learning-notes ch10.2; "Flash Attention V1/V2/V3" explainer;
"5.4 FlashAttention (1/2/3)" reading notes):

* :func:`attn_fwd` / :func:`attn_fwd_rows` -- the definition of section 10.2.1
  (safe softmax with the row max, O = P V) with the 1/sqrt(d)-style scale of
  section 10.2.3 as an argument; LSE = m + ln l.  Optional additive bias on
  the scaled scores (the explainer's V2 section merges mask and bias into the
  score stage): s = scale q.k + bias, -inf masks a key; a row with no finite
  score gets O = 0 and LSE = -inf.
* :func:`attn_bwd` -- the gradients of section 10.2.4 (dV = P^T dO,
  dP = dO V^T, dS = P o (dP - delta), dQ = dS K, dK = dS^T Q) with the scale
  restored by the chain rule; the optional bias enters P as in the forward
  (it is an input: no gradient is formed for it).
* :func:`tiled_fwd` -- the tile update of section 10.2.2 (m~, P~, l~, alpha,
  beta, normalised O') in the FA1 loop order of section 10.2.5.
* :func:`tiled_bwd` -- the recompute backward of section 10.2.4 from the saved
  m and l, with delta_i = dO_i . O_i.
* :func:`decode_bf16`, :func:`decode_e4m3fn` -- exact decoders of the storage
  formats (bfloat16; OCP float8 e4m3fn times its per-tensor scale).
* :func:`decode_mx_e4m3fn` -- e4m3fn codes times their block's power-of-two
  (e8m0) scale: the finer-grained FP8 scaling the explainer's V3 section
  names, in the microscaling layout (32 consecutive elements per block).

Every function is pinned by tests that do not use this module's own
arithmetic: brute force on tiny inputs, closed forms, invariants, finite
differences, torch float64 autograd, and the tiled forms against the naive
ones.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_long)
_L = ctypes.c_long


def build(force: bool = True) -> str:
    """Compile fa_oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
        ):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_attn_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                        ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_fwd_bias.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                             ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_fwd_rows_bias.argtypes = [_dp, _dp, _dp, _dp, _L, _L, ctypes.c_double,
                                                  ctypes.c_int, _lp, _L, _dp, _dp, ctypes.c_int]
        lib.oracle_attn_bwd_bias.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _L, _L,
                                             _L, _L, ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_fwd_rows.argtypes = [_dp, _dp, _dp, _L, _L, ctypes.c_double,
                                             ctypes.c_int, _lp, _L, _dp, _dp, ctypes.c_int]
        lib.oracle_attn_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                        ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.oracle_tiled_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                         ctypes.c_double, ctypes.c_int, _L, _L]
        lib.oracle_tiled_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                         _dp, _L, _L, _L, _L, ctypes.c_double, ctypes.c_int,
                                         _L, _L]
        lib.oracle_decode_bf16.argtypes = [ctypes.POINTER(ctypes.c_ushort), _dp, _L]
        lib.oracle_decode_e4m3fn.argtypes = [ctypes.POINTER(ctypes.c_ubyte), ctypes.c_double,
                                             _dp, _L]
        for name in ("oracle_attn_fwd", "oracle_attn_fwd_rows", "oracle_attn_bwd",
                     "oracle_attn_fwd_bias", "oracle_attn_fwd_rows_bias",
                     "oracle_attn_bwd_bias", "oracle_tiled_fwd", "oracle_tiled_bwd"):
            getattr(lib, name).restype = ctypes.c_int
        lib.oracle_decode_bf16.restype = None
        lib.oracle_decode_e4m3fn.restype = None
        _lib = lib
        return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _shape4(q):
    if q.ndim != 4:
        raise ValueError("expected a [B, H, N, d] array")
    return q.shape


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"{name} returned {rc}")


def _bias4(bias, B, H, N):
    """An additive bias broadcast to a contiguous float64 [B, H, N, N] array."""
    return _f64(np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, H, N, N)))


def attn_fwd(q, k, v, scale: float, causal: bool, nthreads: int | None = None, bias=None):
    """Naive forward by definition.  Returns (O [B,H,N,d], LSE [B,H,N]) in float64.

    bias: None, or an array broadcastable to [B, H, N, N] added to the scaled
    scores (-inf masks a key)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N), dtype=np.float64)
    nt = nthreads or default_threads()
    if bias is None:
        rc = lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                 float(scale), int(bool(causal)), nt)
    else:
        b = _bias4(bias, B, H, N)
        rc = lib.oracle_attn_fwd_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(b), _ptr(o), _ptr(lse),
                                      B, H, N, d, float(scale), int(bool(causal)), nt)
    _check(rc, "oracle_attn_fwd")
    return o, lse


def attn_fwd_rows(q_head, k_head, v_head, rows, scale: float, causal: bool,
                  nthreads: int | None = None, bias_rows=None):
    """Selected rows of ONE head ([N, d] inputs).  Returns (O rows [R, d], LSE rows [R]).

    bias_rows: None, or the [R, N] bias of the selected rows."""
    lib = _load()
    q, k, v = _f64(q_head), _f64(k_head), _f64(v_head)
    N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, d), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    b = None if bias_rows is None else _f64(np.broadcast_to(bias_rows, (rows.size, N)))
    _check(lib.oracle_attn_fwd_rows_bias(_ptr(q), _ptr(k), _ptr(v),
                                         None if b is None else _ptr(b), N, d, float(scale),
                                         int(bool(causal)), rows.ctypes.data_as(_lp), rows.size,
                                         _ptr(o), _ptr(lse), nthreads or default_threads()),
           "oracle_attn_fwd_rows")
    return o, lse


def attn_bwd(q, k, v, dout, scale: float, causal: bool, nthreads: int | None = None,
             bias=None):
    """Naive backward by definition.  Returns (dQ, dK, dV) in float64.

    bias: as for attn_fwd (an input; no gradient is formed for it)."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = _shape4(q)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    b = None if bias is None else _bias4(bias, B, H, N)
    _check(lib.oracle_attn_bwd_bias(_ptr(q), _ptr(k), _ptr(v), None if b is None else _ptr(b),
                                    _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                    float(scale), int(bool(causal)),
                                    nthreads or default_threads()), "oracle_attn_bwd")
    return dq, dk, dv


def tiled_fwd(q, k, v, scale: float, causal: bool, Br: int, Bc: int):
    """Tiled online-softmax forward (FA1 form).  Returns (O, LSE, m, l)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _shape4(q)
    o = np.zeros_like(q)
    lse, m, l = (np.zeros((B, H, N), dtype=np.float64) for _ in range(3))
    _check(lib.oracle_tiled_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(m),
                                _ptr(l), B, H, N, d, float(scale), int(bool(causal)),
                                int(Br), int(Bc)), "oracle_tiled_fwd")
    return o, lse, m, l


def tiled_bwd(q, k, v, o, dout, m, l, scale: float, causal: bool, Br: int, Bc: int):
    """Tiled recompute backward.  Returns (dQ, dK, dV, delta)."""
    lib = _load()
    q, k, v, o, dout, m, l = (_f64(x) for x in (q, k, v, o, dout, m, l))
    B, H, N, d = _shape4(q)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    delta = np.zeros((B, H, N), dtype=np.float64)
    _check(lib.oracle_tiled_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(m),
                                _ptr(l), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), B, H, N,
                                d, float(scale), int(bool(causal)), int(Br), int(Bc)),
           "oracle_tiled_bwd")
    return dq, dk, dv, delta


def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_decode_bf16(b.ctypes.data_as(ctypes.POINTER(ctypes.c_ushort)), _ptr(out),
                           b.size)
    return out


def decode_e4m3fn(codes, scale: float = 1.0) -> np.ndarray:
    """OCP e4m3fn codes (uint8) times a per-tensor scale -> exact float64 values."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib.oracle_decode_e4m3fn(c.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)), float(scale),
                             _ptr(out), c.size)
    return out


def decode_mx_e4m3fn(codes, scales, axis: int) -> np.ndarray:
    """e4m3fn codes with e8m0 block scales -> exact float64 values.

    Element i along `axis` belongs to block i // 32 and is decode(code) *
    2^(E - 127), E the block's scale byte (scales has that axis of length
    ceil(n / 32)).  Multiplying by a power of two is exact in float64.
    """
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    e = np.ascontiguousarray(scales, dtype=np.uint8)
    ax = axis % c.ndim
    n = c.shape[ax]
    if e.shape[ax] != (n + 31) // 32:
        raise ValueError("scales must have ceil(n/32) blocks along axis")
    expanded = np.repeat(e.astype(np.int64) - 127, 32, axis=ax)
    expanded = np.take(expanded, np.arange(n), axis=ax)
    return np.ldexp(decode_e4m3fn(c), expanded)
