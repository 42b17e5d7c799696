"""fa_bwd_noalloc (delta in the library's per-GPU scratch) against fa_bwd
(delta in a caller's workspace) through the C ABI: the same kernels on the
same inputs, so every output must agree bitwise -- on two calls in a row, the
second with a smaller problem (the scratch keeps the first call's contents),
for bf16 and float32, both masks."""
import math

import pytest

import fa_inputs
from _util import run_fwd, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_11_amd as fa  # noqa: E402  (loads libfa.so; fails loudly if missing)


def both_backwards(shape, dtype, causal, seed):
    B, H, N, d = shape
    scale = 1 / math.sqrt(d)
    inp = fa_inputs.make_inputs(shape, dtype, seed=seed)
    (q, k, v), o, lse = run_fwd(inp, scale, causal)
    do = to_device(inp.dout, dtype)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    ref = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_bwd(q, k, v, o, do, lse, *ref, ws, scale, causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, scale, causal)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_workspace_backward(dtype, causal):
    d = 128 if dtype == "bf16" else 64
    for shape in ((2, 3, 1000, d), (1, 2, 129, d)):  # the second call is smaller
        say(f"noalloc {dtype} causal={causal} shape={shape}")
        ref, got = both_backwards(shape, dtype, causal, seed=sum(shape))
        for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.isfinite(r.float()).all(), name
            assert torch.equal(r, g), f"{name} differs from fa_bwd"


def test_noalloc_on_a_side_stream_and_at_the_largest_size():
    """Launches follow the stream passed in; B*H*N = FA_NOALLOC_MAX_ROWS is
    accepted and one more row is refused."""
    B, H, N, d = 1, 512, fa.FA_NOALLOC_MAX_ROWS // 512, 64
    q, k, v, do = fa_inputs.device_normal_bf16((B, H, N, d), seed=5, count=4)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, 0.125, True)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(q) for _ in range(3)]
    fa.fa_bwd(q, k, v, o, do, lse, *ref, ws, 0.125, True)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, 0.125, True, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    big = torch.empty((1, 1, fa.FA_NOALLOC_MAX_ROWS + 1, 64), dtype=torch.bfloat16,
                      device="cuda")
    lbig = torch.empty((1, 1, fa.FA_NOALLOC_MAX_ROWS + 1), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(big, big, big, big, big, lbig, big, big, big, 0.125, False)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
