"""The backward's stage entry points (fa_bwd_delta, fa_bwd_dq, fa_bwd_dkdv)
against fa_bwd, through the C ABI.

Run in fa_bwd's order they give exactly fa_bwd's outputs (the same kernels,
bitwise).  The bf16 dQ stage forms delta_i = dO_i . O_i (FA1 page, section
10.2.4) itself and writes it to the workspace: it must match the definition on
the O the GPU wrote (float32 rounding) and the delta stage's value, and dK/dV
computed from either delta agree to bf16 rounding."""
import math

import numpy as np
import pytest

import fa_inputs
from _util import exact_values, say, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_11_amd as fa  # noqa: E402


def setup(shape, dtype, seed, causal):
    inp = fa_inputs.make_inputs(shape, dtype, seed=seed)
    q, k, v, do = (to_device(x, dtype) for x in (inp.q, inp.k, inp.v, inp.dout))
    B, H, N, d = shape
    scale = 1 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    return inp, (q, k, v, o, do, lse), scale


def new_outputs(q):
    B, H, N, d = q.shape
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    ws.view(torch.float32)[: B * H * N].fill_(float("nan"))
    return grads, ws


def delta_of(ws, q):
    B, H, N, _ = q.shape
    return ws[: B * H * N * 4].view(torch.float32).view(B, H, N)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_stages_in_order_equal_fa_bwd(dtype, d, causal):
    inp, (q, k, v, o, do, lse), scale = setup((2, 3, 300, d), dtype, 17 + d, causal)
    (g1, ws1), (g2, ws2) = new_outputs(q), new_outputs(q)
    fa.fa_bwd(q, k, v, o, do, lse, *g1, ws1, scale, causal)
    order = ([fa.fa_bwd_dq, fa.fa_bwd_dkdv] if dtype == "bf16"
             else [fa.fa_bwd_delta, fa.fa_bwd_dkdv, fa.fa_bwd_dq])
    for stage in order:
        stage(q, k, v, o, do, lse, *g2, ws2, scale, causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        assert torch.equal(a, b), f"{dtype} d={d} causal={causal}: staged {name} differs"
    assert torch.equal(delta_of(ws1, q), delta_of(ws2, q))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 200, 513])
def test_bf16_dq_stage_writes_delta(d, N):
    inp, (q, k, v, o, do, lse), scale = setup((1, 2, N, d), "bf16", 3 * N + d, True)
    (g1, ws1), (g2, ws2) = new_outputs(q), new_outputs(q)
    fa.fa_bwd_dq(q, k, v, o, do, lse, *g1, ws1, scale, True)
    fa.fa_bwd_delta(q, k, v, o, do, lse, *g2, ws2, scale, True)
    torch.cuda.synchronize()
    d_dq, d_stage = to_f64(delta_of(ws1, q)), to_f64(delta_of(ws2, q))
    d_ref = np.sum(to_f64(o) * exact_values(inp.dout, "bf16"), axis=-1)
    den = max(float(np.max(np.abs(d_ref))), 1e-30)
    for tag, got in (("dQ stage", d_dq), ("delta stage", d_stage)):
        assert np.isfinite(got).all(), tag
        e = float(np.max(np.abs(got - d_ref))) / den
        say(f"N={N} d={d} delta from the {tag}: rel err {e:.3e}")
        assert e < 1e-5, tag


def test_dkdv_from_either_delta():
    inp, (q, k, v, o, do, lse), scale = setup((2, 2, 700, 128), "bf16", 5, True)
    (g1, ws1), (g2, ws2) = new_outputs(q), new_outputs(q)
    fa.fa_bwd_dq(q, k, v, o, do, lse, *g1, ws1, scale, True)
    fa.fa_bwd_dkdv(q, k, v, o, do, lse, *g1, ws1, scale, True)
    fa.fa_bwd_delta(q, k, v, o, do, lse, *g2, ws2, scale, True)
    fa.fa_bwd_dkdv(q, k, v, o, do, lse, *g2, ws2, scale, True)
    torch.cuda.synchronize()
    for name, a, b in (("dK", g1[1], g2[1]), ("dV", g1[2], g2[2])):
        a64, b64 = to_f64(a), to_f64(b)
        e = float(np.max(np.abs(a64 - b64))) / float(np.max(np.abs(b64)))
        say(f"{name} from the dQ stage's delta vs the delta stage's: rel {e:.3e}")
        assert e <= 1e-2, name
    assert torch.equal(g1[2], g2[2]), "dV does not depend on delta"
