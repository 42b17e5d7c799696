"""Seeded synthetic inputs for the attention path.

This module is shared by the tests, the smoke check and the benchmark, and it
holds none of the attention arithmetic: it draws the N(0, 1) tensors and casts
them to the storage formats the library takes.  Both the oracle and the HIP
path consume exactly what it returns.

Recipe (the same for every workload): numpy ``default_rng(seed)`` (PCG64)
draws float32 standard normals for Q, K, V and then dO, in that order, each of
shape [B, H, N, d] with d innermost.  The pages' own examples use N(0, 1)
inputs (torch.randn in "FlashAttention-1: eliminating IO", sections 10.2.3 and
10.2.4; np.random.randn with seed 42 in the V1/V2/V3 explainer's Python demo).

Storage formats:
* fp32 -- the draws as they are.
* bf16 -- round-to-nearest-even of each float32 (torch's cast), kept as raw
  uint16 bit patterns so nothing downstream depends on a torch dtype.
* fp8  -- OCP float8 e4m3fn with one scale per tensor, s = amax|X| / 448, and
  codes = round-to-nearest-even(X / s) saturated to +-448.  The explainer says
  only that FP8 inputs are paired with scaling factors (V3 section); the
  per-tensor amax form is the plainest reading.

Additive biases (:func:`draw_bias`): float32 arrays in a row-pitched layout,
values N(0, 1) from their own seed, with -inf entries where a mask is wanted.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp32" | "bf16" | "fp8"
    causal: bool
    backward: bool      # does the workload include the backward pass
    scale: float

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


def _w(name, B, H, N, d, dtype, causal, backward):
    return Workload(name, B, H, N, d, dtype, causal, backward, 1.0 / math.sqrt(d))


# The five workloads: shapes, formats, mask and passes.
WORKLOADS = {
    "fp32_fwdbwd_b1h1n128d64": _w("fp32_fwdbwd_b1h1n128d64", 1, 1, 128, 64, "fp32", False, True),
    "bf16_fwd_b4h16n2048d64": _w("bf16_fwd_b4h16n2048d64", 4, 16, 2048, 64, "bf16", False, False),
    "bf16_causal_fwd_b2h32n8192d128": _w("bf16_causal_fwd_b2h32n8192d128", 2, 32, 8192, 128,
                                          "bf16", True, False),
    "bf16_causal_fwdbwd_b2h16n4096d128": _w("bf16_causal_fwdbwd_b2h16n4096d128", 2, 16, 4096,
                                             128, "bf16", True, True),
    "fp8_fwd_b1h32n16384d128": _w("fp8_fwd_b1h32n16384d128", 1, 32, 16384, 128, "fp8", False,
                                  False),
}


def draw_f32(shape, seed: int = 42, count: int = 4):
    """Draw `count` float32 N(0,1) tensors of `shape` in the order Q, K, V, dO."""
    rng = np.random.default_rng(seed)
    size = int(np.prod(shape))
    return [rng.standard_normal(size, dtype=np.float32).reshape(shape) for _ in range(count)]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_e4m3fn(x: np.ndarray):
    """float32 -> (e4m3fn codes as uint8, per-tensor scale s as a Python float).

    s = amax|x| / 448 computed in float32 (1.0 for an all-zero tensor);
    codes = RNE(x / s) saturated to +-448.  The decoded value of a code times
    s (exact in float64) is what the oracle consumes and what the kernel sees.
    """
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    y = torch.from_numpy(x / s).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, float(s)


def quantize_mx_e4m3fn(x: np.ndarray, axis: int):
    """float32 -> (e4m3fn codes, e8m0 block scales) with blocks of 32
    consecutive elements along `axis` (OCP microscaling convention).

    Per block: amax = max |x|; shared scale 2^(floor(log2 amax) - 8) (8 is the
    largest e4m3 exponent), stored as the byte floor(log2 amax) - 8 + 127
    clipped to [0, 254] (0 for an all-zero block); codes = RNE(x / scale)
    saturated to +-448.  `axis` must have a length that is a multiple of 32 or
    is padded with zeros to one (the padding is dropped from the codes).
    Returns codes shaped like x and scales with that axis divided by 32
    (rounded up) -- the layout fa_fwd_mxfp8 takes.
    """
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    ax = axis % x.ndim
    n = x.shape[ax]
    nb = (n + 31) // 32
    pad = [(0, 0)] * x.ndim
    pad[ax] = (0, nb * 32 - n)
    xp = torch.from_numpy(np.pad(x, pad) if nb * 32 != n else x).movedim(ax, -1)
    xb = xp.reshape(*xp.shape[:-1], nb, 32)
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, 1.0))) - 8.0,
                    -127.0)
    code = torch.clamp(e + 127.0, 0, 254).to(torch.uint8)
    scale = torch.ldexp(torch.ones((), dtype=torch.float32), code.to(torch.int32) - 127)
    y = (xb / scale[..., None]).clamp_(-E4M3_MAX, E4M3_MAX)
    q = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*xb.shape[:-2], nb * 32)
    q = q[..., :n].movedim(-1, ax)
    return np.ascontiguousarray(q.numpy()), np.ascontiguousarray(code.movedim(-1, ax).numpy())


@dataclass
class MXInputs:
    """fp8 inputs with e8m0 block scales: q, k, v codes [B,H,N,d]; qs, ks
    [B,H,N,4] (blocks along d in bytes 0 .. d/32-1, the rest 127); vs
    [B,H,ceil(N/32),d] (blocks along N) -- the layout fa_fwd_mxfp8 takes."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    qs: np.ndarray
    ks: np.ndarray
    vs: np.ndarray


def draw_spread_f32(shape, seed: int = 42, spread_log2: float = 0.0):
    """Q, K, V ~ N(0,1) float32 from `seed` (as draw_f32); with spread > 0,
    each row of Q and K and each head-dim channel of V (per batch and head)
    is multiplied by 2^u, u uniform in [-spread, 0] (a second stream of the
    same generator).  Magnitudes only shrink, so the logits stay within the
    unspread range and the softmax stays as well conditioned as there."""
    q, k, v = draw_f32(shape, seed, count=3)
    if spread_log2 > 0:
        rng = np.random.default_rng(seed + 1)
        row = shape[:-1] + (1,)
        chan = shape[:-2] + (1, shape[-1])
        q, k, v = (x * np.exp2(rng.uniform(-spread_log2, 0.0, size=sz)).astype(np.float32)
                   for x, sz in ((q, row), (k, row), (v, chan)))
    return q, k, v


def make_mx_inputs(shape, seed: int = 42, spread_log2: float = 0.0) -> MXInputs:
    """draw_spread_f32's Q, K, V, block-quantized (mx_inputs_from)."""
    return mx_inputs_from(*draw_spread_f32(shape, seed, spread_log2))


def mx_inputs_from(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> MXInputs:
    """float32 Q, K, V block-quantized: Q and K in blocks along the head dim,
    V in blocks along the sequence."""
    (qc, qs), (kc, ks) = quantize_mx_e4m3fn(q, -1), quantize_mx_e4m3fn(k, -1)
    vc, vs = quantize_mx_e4m3fn(v, -2)

    def word(s):  # one 4-byte word per row
        w = np.full(s.shape[:-1] + (4,), 127, np.uint8)
        w[..., :s.shape[-1]] = s
        return w
    return MXInputs(qc, kc, vc, word(qs), word(ks), vs)


@dataclass
class Inputs:
    """Storage-format inputs for one workload.

    q, k, v, dout: numpy arrays in the storage format (float32, uint16 bf16
    bits, or uint8 e4m3fn codes).  descale: per-tensor (q, k, v) scales for
    fp8, else 1.0.  dout is None for forward-only workloads.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dout: np.ndarray | None
    descale: tuple
    dtype: str


def make_inputs(shape, dtype: str, seed: int = 42, with_dout: bool = True) -> Inputs:
    q, k, v, *rest = draw_f32(shape, seed, 4 if with_dout else 3)
    do = rest[0] if rest else None
    if dtype == "fp32":
        return Inputs(q, k, v, do if with_dout else None, (1.0, 1.0, 1.0), dtype)
    if dtype == "bf16":
        return Inputs(to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v),
                      to_bf16_bits(do) if with_dout else None, (1.0, 1.0, 1.0), dtype)
    if dtype == "fp8":
        (cq, sq), (ck, sk), (cv, sv) = (quantize_e4m3fn(t) for t in (q, k, v))
        return Inputs(cq, ck, cv, None, (sq, sk, sv), dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


def device_normal_bf16(shape, seed: int, count: int = 3):
    """`count` bf16 tensors of `shape` on the current GPU, N(0, 1) float32
    draws from torch's seeded device generator rounded to nearest even.  For
    sequences too long to draw on the host in reasonable time; the oracle gets
    the exact values by copying (parts of) these tensors back."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    out = []
    for _ in range(count):
        x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        out.append(x.to(torch.bfloat16))
        del x
    return out


def pitch(n: int) -> int:
    """A row pitch for an n-key bias row: n rounded up to a multiple of 4 (the
    strides the library takes), plus 4 so that the pitch always differs from n."""
    return (n + 3) // 4 * 4 + 4


def draw_bias(lead, N: int, seed: int, kind: str = "dense", p_mask: float = 0.1,
              window: int = 0) -> np.ndarray:
    """A float32 additive bias for N queries and N keys, in a row-pitched
    array whose last axis has pitch(N) entries (entries past N are NaN: never
    read).  `lead` is the leading shape, e.g. (B, H), (1, H) or (1, 1).

    kind:
      "dense"   -- N(0, 1) values, each entry -inf with probability p_mask
      "keypad"  -- shape lead + (1, pitch): 0 for keys below a length drawn per
                   leading index in [1, N], -inf past it (key padding)
      "window"  -- N(0, 1) values, -inf where key < query - window (a sliding
                   window; with a causal mask the attention becomes banded)
    """
    rng = np.random.default_rng(seed)
    P = pitch(N)
    if kind == "keypad":
        lengths = rng.integers(1, N + 1, size=tuple(lead))
        b = np.full(tuple(lead) + (1, P), np.nan, np.float32)
        keys = np.arange(N)
        b[..., 0, :N] = np.where(keys < lengths[..., None], 0.0, -np.inf)
        return b
    b = np.full(tuple(lead) + (N, P), np.nan, np.float32)
    vals = rng.standard_normal(tuple(lead) + (N, N)).astype(np.float32)
    if kind == "dense":
        vals[rng.random(vals.shape) < p_mask] = -np.inf
    elif kind == "window":
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        vals[..., j < i - window] = -np.inf
    else:
        raise ValueError(kind)
    b[..., :N] = vals
    return b

