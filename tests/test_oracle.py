"""Pins for the CPU oracle: nothing here trusts the oracle's own arithmetic.

Each check ties the oracle to something fixed outside it: hand-derived closed
forms (tests/golden), brute force in pure Python on tiny inputs, invariants of
softmax attention, central finite differences, torch float64 autograd, the
pages' own self-tests, and the tiled online-softmax forms of the pages against
the naive definition.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng_arrays(seed, shape, n=4, scale=1.0):
    r = np.random.default_rng(seed)
    return [scale * r.standard_normal(shape) for _ in range(n)]


def relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------- #
# Closed forms derived by hand (tests/golden/closed_form_tiny.json)
# --------------------------------------------------------------------------- #
def test_golden_closed_form():
    with open(os.path.join(GOLDEN, "closed_form_tiny.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v, do = (np.array(c[x], dtype=np.float64)[None, None] for x in
                       ("q", "k", "v", "dout"))
        o, lse = oracle.attn_fwd(q, k, v, c["scale"], c["causal"])
        np.testing.assert_allclose(o[0, 0], c["o"], rtol=0, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], c["lse"], rtol=0, atol=1e-15, err_msg=c["name"])
        dq, dk, dv = oracle.attn_bwd(q, k, v, do, c["scale"], c["causal"])
        for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            np.testing.assert_allclose(got[0, 0], c[key], rtol=0, atol=1e-15,
                                       err_msg=f"{c['name']} {key}")


# --------------------------------------------------------------------------- #
# Brute force on tiny inputs: exp(s) / sum exp(s) with no max shift
# --------------------------------------------------------------------------- #
def brute_fwd(q, k, v, scale, causal):
    N, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(N)]
    lse = [0.0] * N
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        e = {j: math.exp(scale * sum(q[i][c] * k[j][c] for c in range(d))) for j in js}
        z = sum(e.values())
        for j in js:
            for c in range(d):
                o[i][c] += e[j] / z * v[j][c]
        lse[i] = math.log(z)
    return o, lse


@pytest.mark.parametrize("N,d,causal", list(itertools.product([1, 2, 3, 4], [1, 2, 3],
                                                               [False, True])))
def test_brute_force_tiny(N, d, causal):
    q, k, v, _ = rng_arrays(N * 10 + d, (N, d))
    scale = 0.7
    o_b, lse_b = brute_fwd(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    o, lse = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
    np.testing.assert_allclose(o[0, 0], o_b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], lse_b, rtol=1e-13, atol=1e-14)


def test_probabilities_via_basis_values():
    """V = identity rows makes O the probability matrix itself: rows sum to 1,
    entries are non-negative, masked entries are zero, and each entry equals the
    brute-force softmax."""
    N = 6
    for causal in (False, True):
        q, k, _, _ = rng_arrays(3, (N, N))
        v = np.eye(N)
        o, _ = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], 0.4, causal)
        P = o[0, 0]
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (P >= 0).all()
        if causal:
            assert np.all(P[np.triu_indices(N, 1)] == 0)
        pb, _ = brute_fwd(q.tolist(), k.tolist(), v.tolist(), 0.4, causal)
        np.testing.assert_allclose(P, pb, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------- #
# Invariants and special cases
# --------------------------------------------------------------------------- #
def test_single_key_returns_v():
    q, k, v, _ = rng_arrays(5, (2, 3, 1, 16))
    o, lse = oracle.attn_fwd(q, k, v, 0.25, False)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.25 * np.sum(q * k, axis=-1), rtol=1e-15, atol=0)


def test_constant_v_returns_v():
    q, k, _, _ = rng_arrays(6, (1, 2, 37, 8))
    row = np.random.default_rng(1).standard_normal(8)
    v = np.broadcast_to(row, q.shape).copy()
    for causal in (False, True):
        o, _ = oracle.attn_fwd(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, v, rtol=1e-14, atol=1e-15)


def test_causal_first_row_returns_v0():
    q, k, v, _ = rng_arrays(7, (2, 2, 19, 8), scale=3.0)
    o, lse = oracle.attn_fwd(q, k, v, 0.35, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.35 * np.sum(q[:, :, 0] * k[:, :, 0], -1),
                               rtol=1e-15)


def test_zero_queries_give_means():
    _, k, v, _ = rng_arrays(8, (1, 1, 23, 5))
    q = np.zeros_like(k)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (23, 5)), rtol=1e-13)
    np.testing.assert_allclose(lse, math.log(23), rtol=1e-15)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, 24)[:, None]
    np.testing.assert_allclose(o[0, 0], prefix, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 24)), rtol=1e-14, atol=0)


def test_common_key_shift():
    """Adding one vector c to every key shifts each row's scores by scale q_i.c:
    softmax is unchanged and LSE moves by exactly that amount."""
    q, k, v, _ = rng_arrays(9, (1, 2, 31, 8))
    c = np.random.default_rng(2).standard_normal(8)
    for causal in (False, True):
        o1, l1 = oracle.attn_fwd(q, k, v, 0.3, causal)
        o2, l2 = oracle.attn_fwd(q, k + c, v, 0.3, causal)
        np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l2 - l1, 0.3 * q @ c, rtol=1e-11, atol=1e-12)


def test_joint_key_value_permutation():
    q, k, v, _ = rng_arrays(10, (1, 1, 40, 8))
    perm = np.random.default_rng(3).permutation(40)
    o1, l1 = oracle.attn_fwd(q, k, v, 0.3, False)
    o2, l2 = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)


def test_heads_are_independent_and_ordered():
    """Each (b, h) slice is its own attention problem (no head or batch mixing)."""
    q, k, v, _ = rng_arrays(11, (2, 3, 9, 4))
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    for b, h in itertools.product(range(2), range(3)):
        ob, lb = oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                 v[b:b + 1, h:h + 1], 0.5, True)
        np.testing.assert_array_equal(o[b, h], ob[0, 0])
        np.testing.assert_array_equal(lse[b, h], lb[0, 0])


def test_large_scores_do_not_overflow():
    q, k, v, _ = rng_arrays(12, (1, 1, 16, 8), scale=60.0)
    o, lse = oracle.attn_fwd(q, k, v, 1.0, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    pb = np.zeros_like(o[0, 0])
    s = q[0, 0] @ k[0, 0].T
    for i in range(16):  # exact arithmetic in the shifted form, independent of the oracle
        w = np.exp(s[i] - s[i].max())
        pb[i] = (w / w.sum()) @ v[0, 0]
    np.testing.assert_allclose(o[0, 0], pb, rtol=1e-10, atol=1e-12)


def test_rows_entry_matches_full():
    q, k, v, _ = rng_arrays(13, (1, 1, 50, 16))
    rows = np.array([0, 1, 17, 49, 25])
    for causal in (False, True):
        o, lse = oracle.attn_fwd(q, k, v, 0.25, causal)
        orow, lrow = oracle.attn_fwd_rows(q[0, 0], k[0, 0], v[0, 0], rows, 0.25, causal)
        np.testing.assert_array_equal(orow, o[0, 0, rows])
        np.testing.assert_array_equal(lrow, lse[0, 0, rows])


def test_torch_float64_reference_forward():
    torch = pytest.importorskip("torch")
    q, k, v, _ = rng_arrays(14, (2, 2, 70, 16))
    for causal in (False, True):
        o, lse = oracle.attn_fwd(q, k, v, 0.25, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        s = 0.25 * tq @ tk.transpose(-1, -2)
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(70, 70, dtype=torch.bool), 1), float("-inf"))
        ot = torch.softmax(s, dim=-1) @ tv
        np.testing.assert_allclose(o, ot.numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13)


# --------------------------------------------------------------------------- #
# The pages' tiled online-softmax forms against the definition
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("N", [1, 33, 100, 128])
@pytest.mark.parametrize("blocks", [(1, 1), (7, 7), (32, 32), (128, 128), (16, 40), (64, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_forward_matches_definition(N, blocks, causal):
    q, k, v, _ = rng_arrays(N + blocks[0], (1, 2, N, 8), scale=1.5)
    o, lse = oracle.attn_fwd(q, k, v, 0.3, causal)
    ot, lt, m, l = oracle.tiled_fwd(q, k, v, 0.3, causal, *blocks)
    assert relerr(ot, o) <= 1e-12
    np.testing.assert_allclose(lt, lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m + np.log(l), lse, rtol=1e-12, atol=1e-12)


def test_explainer_numpy_selftest():
    """The explainer's demo: seed 42, n=128, d=16, blocks of 32, error < 1e-6."""
    with open(os.path.join(GOLDEN, "pages_selftests.json")) as f:
        t = json.load(f)["explainer_numpy_demo"]
    np.random.seed(t["seed"])
    n, d = t["n"], t["d"]
    Q, K, V = (np.random.randn(n, d) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o_naive, _ = oracle.attn_fwd(Q[None, None], K[None, None], V[None, None], scale, False)
    o_tiled, _, _, _ = oracle.tiled_fwd(Q[None, None], K[None, None], V[None, None], scale,
                                        False, t["block"], t["block"])
    assert np.abs(o_tiled - o_naive).max() < t["max_err_bound"]


def test_fp32_error_magnitude_matches_pages():
    """An independent float32 implementation (torch) differs from the float64
    oracle by the magnitude the FA1 page prints for float32 (~2e-7 to 3e-7)."""
    torch = pytest.importorskip("torch")
    with open(os.path.join(GOLDEN, "pages_selftests.json")) as f:
        g = json.load(f)
    N, d = g["fa1_forward_example"]["N"], g["fa1_forward_example"]["d"]
    q, k, v, do = (x.astype(np.float32) for x in rng_arrays(15, (N, d)))
    scale = 1.0 / math.sqrt(d)
    o, _ = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], scale, False)
    dq, dk, dv = oracle.attn_bwd(q[None, None], k[None, None], v[None, None], do[None, None],
                                 scale, False)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    ot = torch.softmax((tq @ tk.T) * scale, dim=1) @ tv
    ot.backward(torch.from_numpy(do))
    bound = 20 * g["fa1_forward_example"]["printed_max_abs_err_fp32"]
    assert np.abs(ot.detach().numpy() - o[0, 0]).max() < bound
    for t, ref, key in ((tq, dq, "dq"), (tk, dk, "dk"), (tv, dv, "dv")):
        pb = 20 * g["fa1_backward_example"]["printed_max_abs_err_fp32"][key]
        assert np.abs(t.grad.numpy() - ref[0, 0]).max() < pb, key


# --------------------------------------------------------------------------- #
# Backward
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """Central differences of L = sum(dO o O) for every input element."""
    N, d = 5, 3
    q, k, v, do = rng_arrays(16 + causal, (1, 1, N, d))
    scale = 0.8
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, scale, causal)
        return float(np.sum(do * o))

    h = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in itertools.product(range(N), range(d)):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][(0, 0) + idx] += h
            lp = loss(*args)
            args[which][(0, 0) + idx] -= 2 * h
            lm = loss(*args)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[(0, 0) + idx]) < 1e-8, (which, idx, fd, grad[(0, 0) + idx])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sum_rules(causal):
    """Rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    sum_j dV_j = sum_i dO_i."""
    q, k, v, do = rng_arrays(18, (2, 2, 45, 8))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.35, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    q, k, v, do = rng_arrays(19, (1, 3, 64, 16))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.25, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    s = 0.25 * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(64, 64, dtype=torch.bool), 1), float("-inf"))
    (torch.softmax(s, dim=-1) @ tv).backward(torch.from_numpy(do))
    for t, ref in ((tq, dq), (tk, dk), (tv, dv)):
        np.testing.assert_allclose(ref, t.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("N", [1, 29, 96])
@pytest.mark.parametrize("blocks", [(1, 1), (7, 7), (32, 32), (16, 40)])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_backward_matches_definition(N, blocks, causal):
    q, k, v, do = rng_arrays(20 + N, (1, 2, N, 8))
    o, _, m, l = oracle.tiled_fwd(q, k, v, 0.3, causal, *blocks)
    dq, dk, dv, delta = oracle.tiled_bwd(q, k, v, o, do, m, l, 0.3, causal, *blocks)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, 0.3, causal)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(delta, np.sum(do * o, axis=-1), rtol=1e-14, atol=1e-15)


def test_backward_threading_is_deterministic():
    q, k, v, do = rng_arrays(21, (1, 2, 200, 16))
    a = oracle.attn_bwd(q, k, v, do, 0.25, True, nthreads=1)
    b = oracle.attn_bwd(q, k, v, do, 0.25, True, nthreads=7)
    c = oracle.attn_bwd(q, k, v, do, 0.25, True, nthreads=7)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(y, z)


# --------------------------------------------------------------------------- #
# Exact decoders
# --------------------------------------------------------------------------- #
def test_decode_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode_bf16(bits)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_decode_e4m3fn_all_codes():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode_e4m3fn(codes, 1.0)
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF only; no infinities in e4m3fn
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # the format's fixed points: largest finite, smallest subnormal, one
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    np.testing.assert_array_equal(oracle.decode_e4m3fn(codes[:0x7F], 0.375),
                                  0.375 * got[:0x7F])
