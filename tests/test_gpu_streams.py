"""The library launches on the stream it is given, through the C ABI.

fa_fwd / fa_bwd enqueue their kernels on the caller's stream (an explicit
handle, or torch's current stream when none is passed) and never
synchronise: work on a side stream gives bitwise the same results as on the
default stream, and a forward + backward captured in a HIP graph replays
correctly, several times, on inputs changed eagerly between the replays
(checked against an eager run on the same inputs each time).  Only the
library's kernel launches are recorded in the graph."""
import math

import pytest

import fa_inputs
from _util import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_11_amd as fa  # noqa: E402


def make(shape, seed):
    inp = fa_inputs.make_inputs(shape, "bf16", seed=seed)
    q, k, v, do = (to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.dout))
    B, H, N, d = shape
    bufs = dict(o=torch.empty_like(q), lse=torch.empty((B, H, N), dtype=torch.float32, device="cuda"),
                dq=torch.empty_like(q), dk=torch.empty_like(q), dv=torch.empty_like(q),
                ws=torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                               device="cuda"))
    return (q, k, v, do), bufs, 1 / math.sqrt(d)


def run(ins, b, scale, causal, stream=None):
    q, k, v, do = ins
    fa.fa_fwd(q, k, v, b["o"], b["lse"], scale, causal, stream=stream)
    fa.fa_bwd(q, k, v, b["o"], do, b["lse"], b["dq"], b["dk"], b["dv"], b["ws"], scale, causal,
              stream=stream)


def outputs(b):
    return [b[n].clone() for n in ("o", "lse", "dq", "dk", "dv")]


@pytest.mark.parametrize("explicit", [False, True])
def test_side_stream_matches_default_stream(explicit):
    ins, b, scale = make((2, 3, 300, 128), 21)
    run(ins, b, scale, True)
    torch.cuda.synchronize()
    ref = outputs(b)
    for t in b.values():
        t.zero_()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    if explicit:
        run(ins, b, scale, True, stream=side)
    else:
        with torch.cuda.stream(side):
            run(ins, b, scale, True)
    side.synchronize()
    for name, a, r in zip(("O", "LSE", "dQ", "dK", "dV"), outputs(b), ref):
        assert torch.equal(a, r), f"{name} differs on the side stream"


def test_graph_capture_replays():
    ins, b, scale = make((1, 2, 200, 64), 22)
    originals = [x.clone() for x in ins]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        run(ins, b, scale, True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(ins, b, scale, True)
    torch.cuda.synchronize()
    for r in range(3):
        for x, x0 in zip(ins, originals):  # new inputs, written eagerly
            x.copy_(x0 * (1.0 + 0.25 * r) - 0.1 * r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs(b)
        run(ins, b, scale, True)
        torch.cuda.synchronize()
        for name, a, e in zip(("O", "LSE", "dQ", "dK", "dV"), got, outputs(b)):
            assert torch.isfinite(a.float()).all(), f"replay {r}: {name} not finite"
            assert torch.equal(a, e), f"replay {r}: {name} differs from the eager run"
