"""Pins of the oracle's additive bias (the explainer's V2 section merges mask
and bias into the score stage): s_ij = scale q_i.k_j + bias_ij, a bias of
-inf masks a key, and a row with no finite score has O = 0 and LSE = -inf.

Each check fixes the biased oracle to something other than its own
arithmetic: brute force without a max shift, identities that turn a bias into
a change of the inputs of the (separately pinned) unbiased attention, the
causal mask written as a bias, central finite differences of the forward, and
torch float64 autograd."""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def rand_bias(shape, seed, p_mask=0.25):
    """Bias ~ N(0, 2) with a fraction of -inf entries, never a whole row."""
    rng = np.random.default_rng(seed)
    b = 2.0 * rng.standard_normal(shape)
    m = rng.random(shape) < p_mask
    m[..., 0] = False  # key 0 stays visible in every row (also under the causal mask)
    b[m] = -np.inf
    return b


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_without_max_shift(causal):
    B, H, N, d, scale = 1, 2, 4, 3, 0.7
    q, k, v = rand((B, H, N, d), 1), rand((B, H, N, d), 2), rand((B, H, N, d), 3)
    bias = rand_bias((B, H, N, N), 4)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal, bias=bias)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                w, num = 0.0, [0.0] * d
                for j in range(N):
                    if causal and j > i:
                        continue
                    s = scale * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) + bias[b, h, i, j]
                    e = math.exp(s)  # exp(-inf) = 0
                    w += e
                    for c in range(d):
                        num[c] += e * v[b, h, j, c]
                assert lse[b, h, i] == pytest.approx(math.log(w), rel=1e-13, abs=1e-13)
                for c in range(d):
                    assert o[b, h, i, c] == pytest.approx(num[c] / w, rel=1e-12, abs=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_a_per_row_constant_moves_only_the_lse(causal):
    B, H, N, d, scale = 2, 1, 9, 5, 0.4
    q, k, v = rand((B, H, N, d), 5), rand((B, H, N, d), 6), rand((B, H, N, d), 7)
    c = rand((B, H, N, 1), 8) * 3.0
    o0, lse0 = oracle.attn_fwd(q, k, v, scale, causal)
    o1, lse1 = oracle.attn_fwd(q, k, v, scale, causal, bias=np.broadcast_to(c, (B, H, N, N)))
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0 + c[..., 0], rtol=1e-12, atol=1e-12)


def test_a_log_weight_bias_repeats_keys():
    """bias_ij = ln w_j with integer w_j is attention over K, V with key j
    written w_j times."""
    N, d, scale = 7, 4, 0.6
    q, k, v = rand((1, 1, N, d), 9), rand((1, 1, N, d), 10), rand((1, 1, N, d), 11)
    w = np.array([1, 2, 3, 1, 2, 1, 3])
    o1, lse1 = oracle.attn_fwd(q, k, v, scale, False, bias=np.log(w)[None, None, None, :])
    rep = np.repeat(np.arange(N), w)
    kr, vr = k[:, :, rep], v[:, :, rep]
    # queries padded with copies so that the repeated problem is square
    qr = np.concatenate([q, np.zeros((1, 1, rep.size - N, d))], axis=2)
    o2, lse2 = oracle.attn_fwd(qr, kr, vr, scale, False)
    np.testing.assert_allclose(o1, o2[:, :, :N], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse2[:, :, :N], rtol=1e-12, atol=1e-12)


def test_minus_infinity_removes_keys():
    N, d, scale = 8, 3, 0.9
    q, k, v = rand((1, 2, N, d), 12), rand((1, 2, N, d), 13), rand((1, 2, N, d), 14)
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 1], bool)
    bias = np.where(keep, 0.0, -np.inf)[None, None, None, :]
    o1, lse1 = oracle.attn_fwd(q, k, v, scale, False, bias=bias)
    n = int(keep.sum())
    # the reduced problem: the kept keys, and the first n queries in each call
    for start in range(0, N, n):
        rows = np.arange(start, min(start + n, N))
        qq = np.zeros((1, 2, n, d))
        qq[:, :, : rows.size] = q[:, :, rows]
        o2, lse2 = oracle.attn_fwd(qq, k[:, :, keep], v[:, :, keep], scale, False)
        np.testing.assert_allclose(o1[:, :, rows], o2[:, :, : rows.size], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse1[:, :, rows], lse2[:, :, : rows.size], rtol=1e-12)


def test_the_causal_mask_as_a_bias():
    N, d, scale = 11, 4, 0.5
    q, k, v, do = (rand((2, 1, N, d), s) for s in (15, 16, 17, 18))
    tri = np.where(np.tril(np.ones((N, N), bool)), 0.0, -np.inf)
    o1, lse1 = oracle.attn_fwd(q, k, v, scale, False, bias=tri)
    o2, lse2 = oracle.attn_fwd(q, k, v, scale, True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-12, atol=1e-13)
    g1 = oracle.attn_bwd(q, k, v, do, scale, False, bias=tri)
    g2 = oracle.attn_bwd(q, k, v, do, scale, True)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_with_no_visible_key(causal):
    N, d, scale = 6, 3, 0.8
    q, k, v, do = (rand((1, 1, N, d), s) for s in (19, 20, 21, 22))
    bias = rand_bias((1, 1, N, N), 23)
    dead = [2, 5]
    bias[0, 0, dead, :] = -np.inf
    o, lse = oracle.attn_fwd(q, k, v, scale, causal, bias=bias)
    assert np.all(o[0, 0, dead] == 0.0) and np.all(lse[0, 0, dead] == -np.inf)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal, bias=bias)
    assert np.all(dq[0, 0, dead] == 0.0)
    # the dead rows add nothing to dK, dV: same as giving those rows no gradient
    b2, do2 = bias.copy(), do.copy()
    b2[0, 0, dead, :] = 0.0
    do2[0, 0, dead] = 0.0
    _, dk2, dv2 = oracle.attn_bwd(q, k, v, do2, scale, causal, bias=b2)
    np.testing.assert_allclose(dk, dk2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2, rtol=1e-12, atol=1e-13)


def test_rows_form_matches_full_form():
    N, d, scale = 40, 8, 0.3
    q, k, v = (rand((1, 1, N, d), s) for s in (24, 25, 26))
    bias = rand_bias((1, 1, N, N), 27)
    bias[0, 0, 7, :] = -np.inf
    o, lse = oracle.attn_fwd(q, k, v, scale, True, bias=bias)
    rows = np.array([0, 7, 13, 39])
    o_r, lse_r = oracle.attn_fwd_rows(q[0, 0], k[0, 0], v[0, 0], rows, scale, True,
                                      bias_rows=bias[0, 0, rows])
    np.testing.assert_array_equal(o_r, o[0, 0, rows])
    np.testing.assert_array_equal(lse_r, lse[0, 0, rows])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_by_finite_differences(causal):
    N, d, scale, h = 5, 3, 0.6, 1e-6
    q, k, v, do = (rand((1, 1, N, d), s) for s in (28, 29, 30, 31))
    bias = rand_bias((1, 1, N, N), 32)

    def f(q_, k_, v_):
        return float(np.sum(do * oracle.attn_fwd(q_, k_, v_, scale, causal, bias=bias)[0]))

    grads = oracle.attn_bwd(q, k, v, do, scale, causal, bias=bias)
    for which, g in enumerate(grads):
        for idx in np.ndindex(*q.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            assert g[idx] == pytest.approx((fp - fm) / (2 * h), abs=1e-7, rel=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_float64_autograd(causal):
    B, H, N, d, scale = 2, 2, 13, 6, 1 / math.sqrt(6)
    q, k, v, do = (rand((B, H, N, d), s) for s in (33, 34, 35, 36))
    bias = rand_bias((1, H, N, N), 37)  # broadcast over the batch
    o, lse = oracle.attn_fwd(q, k, v, scale, causal, bias=bias)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal, bias=bias)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2) + torch.tensor(bias)
    if causal:
        s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    to = torch.softmax(s, dim=-1) @ tv
    tl = torch.logsumexp(s, dim=-1)
    (to * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, tl.detach().numpy(), rtol=1e-12, atol=1e-12)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_the_bias_matters():
    """The comparisons above can tell a bias from its negation and from no
    bias at all on these sizes (a sign slip or a dropped bias would show)."""
    N, d, scale = 4, 3, 0.7
    q, k, v = rand((1, 1, N, d), 38), rand((1, 1, N, d), 39), rand((1, 1, N, d), 40)
    bias = rand_bias((1, 1, N, N), 41, p_mask=0.0)
    o, _ = oracle.attn_fwd(q, k, v, scale, False, bias=bias)
    wrong_sign, _ = oracle.attn_fwd(q, k, v, scale, False, bias=-bias)
    no_bias, _ = oracle.attn_fwd(q, k, v, scale, False)
    assert np.abs(o - wrong_sign).max() > 1e-3 and np.abs(o - no_bias).max() > 1e-3
