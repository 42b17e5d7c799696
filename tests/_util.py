"""Shared helpers for the GPU parity tests: upload seeded inputs, run the
library through the binding, decode inputs exactly for the oracle, compare."""
from __future__ import annotations

import sys

import numpy as np

import fa_inputs
import oracle

# Tolerances.  float32: absolute max error on every output.  bf16 / fp8: max
# |gpu - oracle| relative to the oracle's output scale, max |oracle| of the
# compared tensor (floored at 1e-3, so an exactly-zero reference -- e.g. dQ and
# dK of a single key -- is held to 2e-5 / 6e-5 absolute).  LSE is float32 in
# every format: |err| <= atol + rtol |LSE_ref| elementwise; the rtol term
# covers the float32 accumulation of large scores in the matrix cores.
TOL = {"fp32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
LSE_TOL = {"fp32": (1e-5, 0.0), "bf16": (1e-3, 1e-5), "fp8": (1e-3, 1e-5)}
SCALE_FLOOR = 1e-3


def say(*a):
    print("[parity]", *a, file=sys.stderr, flush=True)


def torch_dtype(dtype):
    import torch

    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]


def out_dtype(dtype):
    import torch

    return torch.float32 if dtype == "fp32" else torch.bfloat16


def to_device(arr, dtype):
    """Storage-format numpy array -> device tensor of the library's dtype."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def exact_values(arr, dtype, scale=1.0):
    """Storage-format numpy array -> the float64 values the GPU receives."""
    if dtype == "fp32":
        return arr.astype(np.float64)
    if dtype == "bf16":
        return oracle.decode_bf16(arr)
    return oracle.decode_e4m3fn(arr, scale)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_fwd(inp: fa_inputs.Inputs, scale, causal, prefill_nan=True):
    import torch

    import exact_io_aware_11_amd as fa

    q, k, v = (to_device(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    B, H, N, d = inp.q.shape
    o = torch.empty((B, H, N, d), dtype=out_dtype(inp.dtype), device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if prefill_nan:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    fa.fa_fwd(q, k, v, o, lse, scale, causal, descale=inp.descale)
    torch.cuda.synchronize()
    return (q, k, v), o, lse


def run_bwd(dev_qkv, o, lse, inp, scale, causal, prefill_nan=True):
    import torch

    import exact_io_aware_11_amd as fa

    q, k, v = dev_qkv
    B, H, N, d = q.shape
    dout = to_device(inp.dout, inp.dtype)
    grads = [torch.empty_like(q) for _ in range(3)]
    if prefill_nan:
        for g in grads:
            g.fill_(float("nan"))
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    fa.fa_bwd(q, k, v, o, dout, lse, grads[0], grads[1], grads[2], ws, scale, causal)
    torch.cuda.synchronize()
    delta = ws[: B * H * N * 4].view(torch.float32).view(B, H, N)
    return grads, delta


def rows_by_key_chunks(q_rows, rows, scale, chunk, N, fetch):
    """Oracle rows of one head whose keys are too many to hold in float64 at
    once.  For each query row r (causal: keys 0..r), the oracle's forward runs
    on consecutive key chunks of at most `chunk` keys without a mask, and the
    chunk results are merged by the two-partition rule of "FlashAttention-1:
    eliminating IO", section 10.2.2: LSE = ln sum_c exp(LSE_c) and
    O = sum_c exp(LSE_c - LSE) O_c.  fetch(a, b) returns the exact float64 K
    and V rows a..b-1; q_rows[i] is the float64 query of rows[i].  Returns
    (O [R, d], LSE [R])."""
    d = q_rows.shape[1]
    o_out = np.zeros((len(rows), d))
    lse_out = np.zeros(len(rows))
    end = max(rows) + 1
    parts = [[] for _ in rows]
    for a in range(0, min(end, N), chunk):
        b = min(a + chunk, end)
        kc, vc = fetch(a, b)
        for i, r in enumerate(rows):
            if r < a:
                continue
            n = min(b, r + 1) - a
            qbuf = np.zeros((n, d))
            qbuf[0] = q_rows[i]
            o_c, lse_c = oracle.attn_fwd_rows(qbuf, kc[:n], vc[:n], [0], scale, False)
            parts[i].append((o_c[0], lse_c[0]))
    for i, p in enumerate(parts):
        lses = np.array([x[1] for x in p])
        top = lses.max()
        lse = top + np.log(np.sum(np.exp(lses - top)))
        o_out[i] = sum(np.exp(l - lse) * o for o, l in p)
        lse_out[i] = lse
    return o_out, lse_out


def rel_err(got, ref):
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), SCALE_FLOOR))


def abs_err(got, ref):
    return float(np.max(np.abs(got - ref)))


def check(name, got, ref, dtype, lse=False):
    assert np.isfinite(got).all(), f"{name}: non-finite output (unwritten or overflow)"
    if lse:
        atol, rtol = LSE_TOL[dtype]
        excess = float(np.max(np.abs(got - ref) - (atol + rtol * np.abs(ref))))
        e = abs_err(got, ref)
        say(f"{name}: max abs err {e:.3e} (tol {atol:.0e} + {rtol:.0e}|ref|)")
        assert excess <= 0, f"{name}: {e}"
    elif dtype == "fp32":
        e = abs_err(got, ref)
        say(f"{name}: max abs err {e:.3e} (tol {TOL[dtype]:.0e})")
        assert e <= TOL[dtype], f"{name}: {e}"
    else:
        e = rel_err(got, ref)
        say(f"{name}: max err / max|ref| {e:.3e} (tol {TOL[dtype]:.0e})")
        assert e <= TOL[dtype], f"{name}: {e}"
    return e
