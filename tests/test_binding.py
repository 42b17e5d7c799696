"""The Python binding refuses what the C ABI cannot check: host tensors,
wrong shapes and mixed element types never reach a kernel.  (No GPU needed:
every call here raises before the library is called.)"""
import pytest

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_io_aware_11_amd")


def host(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_host_tensors_are_rejected():
    x, lse = host((1, 1, 8, 64)), host((1, 1, 8), torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd(x, x, x, x, lse, 0.125, False)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd_bias(x, x, x, host((1, 1, 8, 8), torch.float32), x, lse, 0.125, False)
    ws = host((256,), torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_bwd(x, x, x, x, x, lse, x, x, x, ws, 0.125, False)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_bwd_bias(x, x, x, host((1, 1, 8, 8), torch.float32), x, x, lse, x, x, x, ws, 0.125,
                       False)
    codes, sc = host((1, 1, 8, 64), torch.uint8), host((1, 1, 8, 4), torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd_mxfp8(codes, codes, codes, sc, sc, host((1, 1, 1, 64), torch.uint8), x, lse,
                        0.125, False)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_bwd_noalloc(x, x, x, x, x, lse, x, x, x, 0.125, False)
    for stage in (fa.fa_bwd_delta, fa.fa_bwd_dkdv, fa.fa_bwd_dq):
        with pytest.raises(ValueError, match="GPU tensor"):
            stage(x, x, x, x, x, lse, x, x, x, ws, 0.125, False)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_std_fwd(x, x, x, x, lse, ws, 0.125, False)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_measure_mfma_rate(host((512,), torch.float32), 1, 1)


def test_flop_counts():
    """The FLOP counts bench.py divides by: 4 B H N^2 d for the forward
    (two products of 2 N^2 d each), 10 for the backward (five), halved under
    the causal mask."""
    assert fa.flops_fwd(2, 3, 128, 64, False) == 4.0 * 2 * 3 * 128 * 128 * 64
    assert fa.flops_fwd(2, 3, 128, 64, True) == 2.0 * 2 * 3 * 128 * 128 * 64
    assert fa.flops_bwd(1, 1, 256, 128, False) == 10.0 * 256 * 256 * 128
    assert fa.flops_bwd(1, 1, 256, 128, True) == 5.0 * 256 * 256 * 128

