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


def full_check_fwd(inp, scale, causal, tag):
    say(f"{tag}: fwd {inp.dtype} shape={inp.q.shape} causal={causal}")
    dev, o, lse = run_fwd(inp, scale, causal)
    qs, ks, vs = (exact_values(x, inp.dtype, s) for x, s in zip((inp.q, inp.k, inp.v), inp.descale))
    o_ref, lse_ref = oracle.attn_fwd(qs, ks, vs, scale, causal)
    check(f"{tag} O", to_f64(o), o_ref, inp.dtype)
    check(f"{tag} LSE", to_f64(lse), lse_ref, inp.dtype, lse=True)
    return dev, o, lse, (qs, ks, vs)


def bf16_inputs_from(q, k, v, do=None):
    return fa_inputs.Inputs(fa_inputs.to_bf16_bits(q), fa_inputs.to_bf16_bits(k),
                            fa_inputs.to_bf16_bits(v),
                            None if do is None else fa_inputs.to_bf16_bits(do), (1., 1., 1.),
                            "bf16")


# Inputs whose largest scores lie far beyond the first key tile of their rows.
#  growing     keys grow along the sequence: each later tile moves the row's
#              reference up
#  jump        a few late keys score ~12 d E|q| above the first tile's maximum,
#              so far that exp against that maximum overflows float32
#  jump_big_v  late keys 2^110 .. 2^126 times the first tile's maximum in
#              probability (finite), their values times 2^20: P V overflows
#              before any rescaling
#  jump_huge_v late keys ~2^40 times it (row sums stay below 2^64), their
#              values times 2^100: P V overflows while the row sum does not
#  jump_early  as jump from key 100 on: under the causal mask with 256-row
#              blocks, the short block of a pair (rows 0..255, processed
#              second) overflows too, not only the long one
OUTGROW_KINDS = ["growing", "jump", "jump_big_v", "jump_huge_v", "jump_early"]


def outgrow_inputs(kind, causal, d, N=700):
    return bf16_inputs_from(*outgrow_f32(kind, causal, d, N))


def outgrow_f32(kind, causal, d, N=700):
    """The float32 Q, K, V, dO behind outgrow_inputs."""
    rng = np.random.default_rng(31 + d + int(causal))
    q = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    if kind == "growing":
        q = np.abs(q) + 0.5
        k = np.abs(k) * np.linspace(0.2, 3.0, N, dtype=np.float32)[None, None, :, None]
    else:
        big = np.arange(100 if kind == "jump_early" else 300, N, 97)  # one per row block or so
        q[...] = np.abs(q) + 1.0
        k[:, :, big, :] = {"jump": 12.0, "jump_early": 12.0,
                           "jump_big_v": 4.3 if d == 128 else 6.1,
                           "jump_huge_v": 1.46 if d == 128 else 2.07}[kind]
        if kind == "jump_big_v":
            v[:, :, big, :] *= 2.0 ** 20
        if kind == "jump_huge_v":
            v[:, :, big, :] *= 2.0 ** 100
    do = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    return q, k, v, do


def sampled_fwd_check(w, heads, rows, seed=42, block=256):
    """The workload at full size in the launch configuration bench.py times:
    `rows` of the listed heads, and in EVERY (b, h) six rows -- the first and
    last rows of the first row block, the first row of the second, a row that
    moves with the head index, and the last two rows -- against the oracle's
    rows (each costs one pass over the head's keys)."""
    inp = fa_inputs.make_inputs(w.shape, w.dtype, seed=seed, with_dout=False)
    dev, o, lse = run_fwd(inp, w.scale, w.causal)
    o_all, lse_all = to_f64(o), to_f64(lse)
    assert np.isfinite(o_all).all() and np.isfinite(lse_all).all()

    def exact_head(b, h):
        return (exact_values(x[b, h], w.dtype, s)
                for x, s in zip((inp.q, inp.k, inp.v), inp.descale))

    for (b, h) in heads:
        o_ref, lse_ref = oracle.attn_fwd_rows(*exact_head(b, h), rows, w.scale, w.causal)
        check(f"{w.name} head ({b},{h}) O rows", o_all[b, h, rows], o_ref, w.dtype)
        check(f"{w.name} head ({b},{h}) LSE rows", lse_all[b, h, rows], lse_ref, w.dtype,
              lse=True)
    worst_o = worst_l = 0.0
    for b in range(w.B):
        for h in range(w.H):
            bh = b * w.H + h
            every = np.unique([0, block - 1, block, (977 * bh + 131) % w.N, w.N - 2, w.N - 1])
            o_ref, lse_ref = oracle.attn_fwd_rows(*exact_head(b, h), every, w.scale, w.causal)
            worst_o = max(worst_o, rel_err(o_all[b, h, every], o_ref))
            atol, rtol = LSE_TOL[w.dtype]
            worst_l = max(worst_l, float(np.max(np.abs(lse_all[b, h, every] - lse_ref)
                                                - (atol + rtol * np.abs(lse_ref)))))
            assert rel_err(o_all[b, h, every], o_ref) <= TOL[w.dtype], (b, h)
    say(f"{w.name}: all {w.B * w.H} heads, 6 rows each: worst O err {worst_o:.3e}, "
        f"worst LSE excess over its bar {worst_l:.3e}")
    assert worst_l <= 0
    return inp, dev, o, lse


def sample_rows(N, n=24, seed=0):
    r = np.random.default_rng(seed).choice(N, size=n, replace=False)
    edge = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 2, N - 1]
    return np.unique(np.concatenate([r, edge]))
