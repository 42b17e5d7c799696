"""GPU parity of the additive bias / general mask path (fa_fwd_bias,
fa_bwd_bias; the explainer's V2 section merges mask and bias into the score
stage) against the float64 oracle with the same bias, through the C ABI.

Bars as for the plain path (float32 1e-5 absolute; bf16 2e-2 of the output
scale; LSE 1e-5 / 1e-3 + 1e-5|LSE|).  Rows that see no finite score must come
out exactly: O = 0, LSE = -inf, dQ = 0.  Biases are row-pitched views (the
pitch is never N), broadcast over batch and/or heads through zero strides."""
import math

import numpy as np
import pytest

import fa_inputs
import oracle
from _util import check, exact_values, out_dtype, say, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_11_amd as fa  # noqa: E402


def bias_views(b_np, N):
    """(device view of the first N keys of each row, float64 values for the oracle)."""
    dev = torch.from_numpy(b_np).cuda()[..., :N]
    return dev, b_np[..., :N].astype(np.float64)


def run_fwd_bias(dev_qkv, bias_dev, scale, causal, dtype):
    q, k, v = dev_qkv
    B, H, N, d = q.shape
    o = torch.full((B, H, N, d), float("nan"), dtype=out_dtype(dtype), device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_bias(q, k, v, bias_dev, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o, lse


def run_bwd_bias(dev_qkv, bias_dev, o, lse, dout, scale, causal):
    q, k, v = dev_qkv
    B, H, N, d = q.shape
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    fa.fa_bwd_bias(q, k, v, bias_dev, o, dout, lse, grads[0], grads[1], grads[2], ws, scale,
                   causal)
    torch.cuda.synchronize()
    return grads


def check_lse(tag, got, ref, dtype):
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), dead), f"{tag}: -inf rows differ"
    if (~dead).any():
        check(tag, got[~dead], ref[~dead], dtype, lse=True)
    return dead


def check_case(inp, b_np, scale, causal, tag, backward=True):
    B, H, N, d = inp.q.shape
    dev = tuple(to_device(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    bias_dev, bias_ref = bias_views(b_np, N)
    say(f"{tag}: fwd")
    o, lse = run_fwd_bias(dev, bias_dev, scale, causal, inp.dtype)
    qs, ks, vs = (exact_values(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    o_ref, lse_ref = oracle.attn_fwd(qs, ks, vs, scale, causal, bias=bias_ref)
    dead = check_lse(f"{tag} LSE", to_f64(lse), lse_ref, inp.dtype)
    o64 = to_f64(o)
    assert np.all(o64[dead] == 0.0), f"{tag}: rows with no finite score must be 0"
    check(f"{tag} O", o64, o_ref, inp.dtype)
    if not backward:
        return
    say(f"{tag}: bwd ({int(dead.sum())} empty rows)")
    dout = to_device(inp.dout, inp.dtype)
    dq, dk, dv = run_bwd_bias(dev, bias_dev, o, lse, dout, scale, causal)
    dos = exact_values(inp.dout, inp.dtype)
    rq, rk, rv = oracle.attn_bwd(qs, ks, vs, dos, scale, causal, bias=bias_ref)
    dq64 = to_f64(dq)
    assert np.all(dq64[dead] == 0.0)
    check(f"{tag} dQ", dq64, rq, inp.dtype)
    check(f"{tag} dK", to_f64(dk), rk, inp.dtype)
    check(f"{tag} dV", to_f64(dv), rv, inp.dtype)


def dense_bias(B, H, N, seed):
    """[B, H, N, pitch] N(0,1) with 10 % -inf, and a few rows masked entirely."""
    b = fa_inputs.draw_bias((B, H), N, seed, "dense")
    b[0, H - 1, : max(1, N // 7), :N] = -np.inf      # a run of empty rows at the top
    b[B - 1, 0, N - 1, :N] = -np.inf                 # and the last row
    return b


@pytest.mark.parametrize("N", [1, 65, 257, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_dense_bias(N, d, causal):
    inp = fa_inputs.make_inputs((2, 3, N, d), "bf16", seed=5 * N + d)
    check_case(inp, dense_bias(2, 3, N, seed=N + d), 1 / math.sqrt(d), causal,
               f"bf16 dense bias 2x3x{N}x{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("at", [5, 100, 400])
def test_bf16_bias_that_jumps(at, causal, d):
    """A bias column of +200 at one key (and +150 on a later one): every row
    that sees it has its maximum there, far above the scores of its first
    tile, so the reference max must move before those probabilities are
    formed (the SAFE path's lazy rescale); at key 5 the jump lies in the
    first tile itself."""
    N = 700
    inp = fa_inputs.make_inputs((1, 2, N, d), "bf16", seed=at + d)
    b = fa_inputs.draw_bias((1, 2), N, seed=at, kind="dense", p_mask=0.0)
    b[..., :, at] = 200.0
    b[..., :, min(at + 333, N - 1)] = 150.0
    check_case(inp, b, 1 / math.sqrt(d), causal, f"bf16 jumping bias at {at} d={d}")


@pytest.mark.parametrize("N", [31, 32, 33, 63, 64, 96, 97, 129])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_bias_tile_boundaries(N, causal):
    """Sequence lengths at and around the key-tile widths of the bias kernels
    (32-key tiles in the d = 128 forward, 64-key tiles elsewhere)."""
    d = 128
    inp = fa_inputs.make_inputs((1, 2, N, d), "bf16", seed=7 * N + int(causal))
    check_case(inp, dense_bias(1, 2, N, seed=11 * N), 1 / math.sqrt(d), causal,
               f"bf16 dense bias 1x2x{N}x{d} causal={causal}")


@pytest.mark.parametrize("N", [65, 1000])
@pytest.mark.parametrize("kind", ["shared", "keypad", "window"])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_broadcast_biases(N, kind, causal):
    d = 128
    inp = fa_inputs.make_inputs((2, 3, N, d), "bf16", seed=3 * N)
    if kind == "shared":      # one [N, N] bias for every batch entry and head
        b = fa_inputs.draw_bias((1, 1), N, seed=N, kind="dense")
    elif kind == "keypad":    # [B, 1, 1, N]: per-batch key lengths
        b = fa_inputs.draw_bias((2, 1), N, seed=N, kind="keypad")
    else:                     # [1, H, N, N] sliding window per head
        b = fa_inputs.draw_bias((1, 3), N, seed=N, kind="window", window=N // 5)
    check_case(inp, b, 1 / math.sqrt(d), causal, f"bf16 {kind} bias 2x3x{N}x{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["shared", "keypad"])
def test_bf16_bias_grouped_order(kind, causal, d):
    """Biases that every head of a batch entry shares (head stride 0) on grids
    where the bf16 forward groups its workgroups by 8 heads x 8 row blocks
    (8 heads per batch entry, 8 blocks or causal pairs of blocks per head):
    every output against the full oracle, forward and backward."""
    N = 2048 if causal else 1024
    B = 2 if kind == "keypad" else 1
    inp = fa_inputs.make_inputs((B, 8, N, d), "bf16", seed=31 * d + int(causal))
    if kind == "shared":      # one [N, N] bias (10 % -inf) for every head
        b = fa_inputs.draw_bias((1, 1), N, seed=d, kind="dense")
    else:                     # [B, 1, 1, N]: per-batch key lengths
        b = fa_inputs.draw_bias((B, 1), N, seed=d, kind="keypad")
    check_case(inp, b, 1 / math.sqrt(d), causal,
               f"bf16 {kind} bias {B}x8x{N}x{d} causal={causal} (grouped order)")


@pytest.mark.parametrize("N", [1, 65, 257])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_dense_bias(N, d, causal):
    inp = fa_inputs.make_inputs((1, 2, N, d), "fp32", seed=9 * N + d)
    check_case(inp, dense_bias(1, 2, N, seed=2 * N + d), 1 / math.sqrt(d), causal,
               f"fp32 dense bias 1x2x{N}x{d} causal={causal}")


def test_mask_as_bias_equals_the_causal_kernel():
    """A lower-triangular 0 / -inf bias with causal = 0 and the causal kernel
    compute the same attention (both checked against each other and the oracle)."""
    N, d = 300, 128
    inp = fa_inputs.make_inputs((1, 2, N, d), "bf16", seed=11)
    tri = np.full((1, 1, N, fa_inputs.pitch(N)), np.nan, np.float32)
    tri[0, 0, :, :N] = np.where(np.tril(np.ones((N, N), bool)), 0.0, -np.inf)
    check_case(inp, tri, 1 / math.sqrt(d), False, "bf16 triangular bias")
    dev = tuple(to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o1, lse1 = run_fwd_bias(dev, bias_views(tri, N)[0], 1 / math.sqrt(d), False, "bf16")
    o2 = torch.empty_like(o1)
    lse2 = torch.empty_like(lse1)
    fa.fa_fwd(*dev, o2, lse2, 1 / math.sqrt(d), True)
    torch.cuda.synchronize()
    check("triangular bias vs causal O", to_f64(o1), to_f64(o2), "bf16")
    check("triangular bias vs causal LSE", to_f64(lse1), to_f64(lse2), "bf16", lse=True)


def test_full_bf16_causal_window_bias_b2h16n4096d128():
    """The fwd+bwd workload's shape with a shared [N, N] bias that also masks a
    sliding window: with the causal mask each query sees its last 1024 keys.
    Whole-head oracle forward and backward on two heads."""
    B, H, N, d = 2, 16, 4096, 128
    inp = fa_inputs.make_inputs((B, H, N, d), "bf16", seed=42)
    b_np = fa_inputs.draw_bias((1, 1), N, seed=7, kind="window", window=1023)
    dev = tuple(to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    bias_dev, bias_ref = bias_views(b_np, N)
    scale = 1 / math.sqrt(d)
    o, lse = run_fwd_bias(dev, bias_dev, scale, True, "bf16")
    dout = to_device(inp.dout, "bf16")
    dq, dk, dv = run_bwd_bias(dev, bias_dev, o, lse, dout, scale, True)
    o64, lse64 = to_f64(o), to_f64(lse)
    assert np.isfinite(o64).all() and np.isfinite(lse64).all()
    g64 = [to_f64(x) for x in (dq, dk, dv)]
    for (b, h) in [(0, 0), (1, 15)]:
        tag = f"window bias 2x16x4096x128 head ({b},{h})"
        qs, ks, vs, dos = (exact_values(x[b:b + 1, h:h + 1], "bf16")
                           for x in (inp.q, inp.k, inp.v, inp.dout))
        o_ref, lse_ref = oracle.attn_fwd(qs, ks, vs, scale, True, bias=bias_ref)
        check(f"{tag} O", o64[b:b + 1, h:h + 1], o_ref, "bf16")
        check(f"{tag} LSE", lse64[b:b + 1, h:h + 1], lse_ref, "bf16", lse=True)
        refs = oracle.attn_bwd(qs, ks, vs, dos, scale, True, bias=bias_ref)
        for name, got, ref in zip(("dQ", "dK", "dV"), g64, refs):
            check(f"{tag} {name}", got[b:b + 1, h:h + 1], ref, "bf16")


def test_full_bf16_causal_bias_fwd_b2h32n8192d128():
    """The headline forward's shape with a shared [N, N] N(0,1) bias carrying
    10 % -inf; sampled rows of two heads against the oracle."""
    B, H, N, d = 2, 32, 8192, 128
    inp = fa_inputs.make_inputs((B, H, N, d), "bf16", seed=42, with_dout=False)
    b_np = fa_inputs.draw_bias((1, 1), N, seed=8, kind="dense")
    dev = tuple(to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    bias_dev, _ = bias_views(b_np, N)
    scale = 1 / math.sqrt(d)
    o, lse = run_fwd_bias(dev, bias_dev, scale, True, "bf16")
    o64, lse64 = to_f64(o), to_f64(lse)
    rows = np.unique(np.concatenate([np.random.default_rng(1).choice(N, 20, replace=False),
                                     [1, 63, 64, 127, 128, N // 2, N - 1]]))
    for (b, h) in [(0, 3), (1, 31)]:
        tag = f"dense bias 2x32x8192x128 head ({b},{h})"
        qs, ks, vs = (exact_values(x[b, h], "bf16") for x in (inp.q, inp.k, inp.v))
        o_ref, lse_ref = oracle.attn_fwd_rows(qs, ks, vs, rows, scale, True,
                                              bias_rows=b_np[0, 0, rows, :N].astype(np.float64))
        dead = check_lse(f"{tag} LSE rows", lse64[b, h, rows], lse_ref, "bf16")
        assert np.all(o64[b, h, rows][dead] == 0.0)
        check(f"{tag} O rows", o64[b, h, rows], o_ref, "bf16")
    # every (b, h) at a few rows: first and last of the first block, one in
    # the middle that moves with the head, the last (the grouped block order)
    for b in range(B):
        for h in range(H):
            few = np.array(sorted({0, 127, 128 + 61 * (b * H + h) % (N - 256), N - 1}))
            qs, ks, vs = (exact_values(x[b, h], "bf16") for x in (inp.q, inp.k, inp.v))
            o_ref, lse_ref = oracle.attn_fwd_rows(qs, ks, vs, few, scale, True,
                                                  bias_rows=b_np[0, 0, few, :N].astype(np.float64))
            tag = f"dense bias 2x32x8192x128 head ({b},{h}) rows {few.tolist()}"
            dead = check_lse(f"{tag} LSE", lse64[b, h, few], lse_ref, "bf16")
            assert np.all(o64[b, h, few][dead] == 0.0)
            check(f"{tag} O", o64[b, h, few], o_ref, "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_longest_sequence_keypad_bias(d, causal):
    """N = 2^17 in one head with a key-padding bias [1,1,1,N] (keys past a
    drawn length masked): the bias kernels' long-sequence offsets and tile
    counts (32-key tiles at d = 128), sampled rows against the oracle,
    including rows past the padding length and the last rows."""
    N = 1 << 17
    inp = fa_inputs.make_inputs((1, 1, N, d), "bf16", seed=d + int(causal), with_dout=False)
    b_np = fa_inputs.draw_bias((1, 1), N, seed=5 + d, kind="keypad")
    dev = tuple(to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    bias_dev, _ = bias_views(b_np, N)
    scale = 1 / math.sqrt(d)
    o, lse = run_fwd_bias(dev, bias_dev, scale, causal, "bf16")
    o64, lse64 = to_f64(o), to_f64(lse)
    rows = np.unique(np.concatenate([np.random.default_rng(d).choice(N, 12, replace=False),
                                     [0, 31, 32, 33, 4095, N - 33, N - 2, N - 1]]))
    qs, ks, vs = (exact_values(x[0, 0], "bf16") for x in (inp.q, inp.k, inp.v))
    o_ref, lse_ref = oracle.attn_fwd_rows(qs, ks, vs, rows, scale, causal,
                                          bias_rows=b_np[0, 0, 0, :N].astype(np.float64))
    tag = f"keypad bias 1x1x{N}x{d} causal={causal}"
    say(f"{tag}: {int(np.isneginf(lse_ref).sum())} of {rows.size} sampled rows empty")
    dead = check_lse(f"{tag} LSE rows", lse64[0, 0, rows], lse_ref, "bf16")
    assert np.all(o64[0, 0, rows][dead] == 0.0)
    check(f"{tag} O rows", o64[0, 0, rows], o_ref, "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_rows_past_the_end_wrap(d, causal):
    """A bias slice at the limit the library accepts: N = 1025 rows with a
    row stride of 1048572 floats, so ((N-1) stride + N) floats fill 4 GiB
    less a few KiB.  The last row block's 127 padding rows (1025..1151) then
    sit past 2^32 bytes: the 32-bit offsets of their bias loads wrap (the
    forward stages bias rows without clamping them, the backward's row offsets
    are formed the same way) and read somewhere inside the slice.  Those rows
    are never written; every real row must still match the oracle, forward
    and backward."""
    N = 1025
    sq = ((2**32 - 4096 - 4 * N) // (4 * (N - 1))) // 4 * 4
    assert (N - 1) * sq * 4 < 2**32 <= N * sq * 4
    inp = fa_inputs.make_inputs((1, 2, N, d), "bf16", seed=17 * d + int(causal))
    dense = fa_inputs.draw_bias((1, 1), N, seed=d, kind="dense")[0, 0, :, :N]
    buf = torch.zeros((N - 1) * sq + N, dtype=torch.float32, device="cuda")
    bias = torch.as_strided(buf, (1, 1, N, N), (0, 0, sq, 1))
    bias[0, 0].copy_(torch.from_numpy(np.ascontiguousarray(dense)))
    scale = 1 / math.sqrt(d)
    dev = tuple(to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    tag = f"bias stride {sq} 1x2x{N}x{d} causal={causal}"
    say(f"{tag}: fwd")
    o, lse = run_fwd_bias(dev, bias, scale, causal, "bf16")
    qs, ks, vs = (exact_values(x, "bf16") for x in (inp.q, inp.k, inp.v))
    bias_ref = dense.astype(np.float64)[None, None]
    o_ref, lse_ref = oracle.attn_fwd(qs, ks, vs, scale, causal, bias=bias_ref)
    dead = check_lse(f"{tag} LSE", to_f64(lse), lse_ref, "bf16")
    assert np.all(to_f64(o)[dead] == 0.0)
    check(f"{tag} O", to_f64(o), o_ref, "bf16")
    say(f"{tag}: bwd")
    dout = to_device(inp.dout, "bf16")
    dq, dk, dv = run_bwd_bias(dev, bias, o, lse, dout, scale, causal)
    rq, rk, rv = oracle.attn_bwd(qs, ks, vs, exact_values(inp.dout, "bf16"), scale, causal,
                                 bias=bias_ref)
    check(f"{tag} dQ", to_f64(dq), rq, "bf16")
    check(f"{tag} dK", to_f64(dk), rk, "bf16")
    check(f"{tag} dV", to_f64(dv), rv, "bf16")
    del buf, bias
    torch.cuda.empty_cache()
