"""GPU parity of the alternative forward schedules (bf16, d = 128, no bias),
selected with FA_FWD_SCHEDULE: "pingpong" (two wave groups per SIMD alternate
matrix products and softmax; the reading notes' three-generation table, FA3
ping-pong scheduling) and "rows64" (64 query rows per wave).  They compute
what the default schedule computes, so the same bars hold: against the
float64 oracle on ragged and multi-tile shapes, on inputs whose scores
outgrow the first key tile, at the full causal B2 H32 N8192 size (every head,
six rows each), plus bitwise determinism and LSE agreement with the default.
"""
import math

import numpy as np
import pytest

import fa_inputs
from _util import (OUTGROW_KINDS, full_check_fwd, outgrow_inputs, run_fwd, sample_rows,
                   sampled_fwd_check, say, to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_11_amd as fa  # noqa: E402,F401  (loads libfa.so; fails loudly if missing)

SCHEDULES = ["pingpong", "rows64"]


@pytest.fixture(params=SCHEDULES)
def schedule(request, monkeypatch):
    monkeypatch.setenv("FA_FWD_SCHEDULE", request.param)
    return request.param


@pytest.mark.parametrize("N", [1, 31, 33, 64, 65, 255, 256, 257, 300, 513, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_schedule_shapes(schedule, N, causal):
    inp = fa_inputs.make_inputs((2, 2, N, 128), "bf16", seed=N + 7, with_dout=False)
    full_check_fwd(inp, 1 / math.sqrt(128), causal, f"{schedule} bf16 2x2x{N}x128")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", OUTGROW_KINDS)
def test_schedule_scores_that_outgrow_the_first_tile(schedule, kind, causal):
    full_check_fwd(outgrow_inputs(kind, causal, 128), 1 / math.sqrt(128), causal,
                   f"{schedule} {kind}")


def test_schedule_full_causal_b2h32n8192d128(schedule):
    w = fa_inputs.WORKLOADS["bf16_causal_fwd_b2h32n8192d128"]
    sampled_fwd_check(w, [(0, 0), (1, 31)], sample_rows(w.N, n=12), block=256)


@pytest.mark.parametrize("causal", [False, True])
def test_schedule_deterministic_and_agrees_with_default(schedule, causal, monkeypatch):
    inp = fa_inputs.make_inputs((2, 4, 1500, 128), "bf16", seed=77, with_dout=False)
    _, o1, l1 = run_fwd(inp, 1 / math.sqrt(128), causal)
    _, o2, l2 = run_fwd(inp, 1 / math.sqrt(128), causal)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    monkeypatch.setenv("FA_FWD_SCHEDULE", "interleaved")
    _, o0, l0 = run_fwd(inp, 1 / math.sqrt(128), causal)
    lse_d = float(np.max(np.abs(to_f64(l1) - to_f64(l0)) / (1 + np.abs(to_f64(l0)))))
    o_d = float(np.max(np.abs(to_f64(o1) - to_f64(o0))) / np.max(np.abs(to_f64(o0))))
    say(f"{schedule} vs interleaved: LSE {lse_d:.2e}, O {o_d:.2e}")
    assert lse_d <= 1e-5 and o_d <= 2 ** -7


@pytest.mark.parametrize("case", ["d64", "bias", "fp8"])
def test_schedule_applies_to_bf16_d128_without_bias_only(schedule, case, monkeypatch):
    """Elsewhere (d = 64, a bias, fp8) the variable is accepted and changes
    nothing: the outputs equal the default's bitwise."""
    causal = True
    if case == "d64":
        inp = fa_inputs.make_inputs((1, 2, 700, 64), "bf16", seed=5, with_dout=False)
    elif case == "fp8":
        inp = fa_inputs.make_inputs((1, 2, 700, 128), "fp8", seed=5, with_dout=False)
    else:
        inp = fa_inputs.make_inputs((1, 2, 700, 128), "bf16", seed=5, with_dout=False)

    def run():
        if case != "bias":
            _, o, lse = run_fwd(inp, 0.1, causal)
            return o, lse
        q, k, v = (torch.from_numpy(x).view(torch.int16).view(torch.bfloat16).cuda()
                   for x in (inp.q, inp.k, inp.v))
        bias = torch.from_numpy(fa_inputs.draw_bias((1, 1), 700, seed=3, kind="dense")).cuda()
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        fa.fa_fwd_bias(q, k, v, bias[..., :700], o, lse, 0.1, causal)
        torch.cuda.synchronize()
        return o, lse

    o1, l1 = run()
    monkeypatch.setenv("FA_FWD_SCHEDULE", "interleaved")
    o0, l0 = run()
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)) and torch.equal(l1, l0)

