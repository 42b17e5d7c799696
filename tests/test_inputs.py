"""The seeded input generators and storage-format casts (CPU only)."""
import numpy as np
import fa_inputs
import oracle


def test_draws_are_seeded_and_ordered():
    a = fa_inputs.draw_f32((2, 3, 5, 4), seed=42, count=4)
    b = fa_inputs.draw_f32((2, 3, 5, 4), seed=42, count=3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert a[0].dtype == np.float32 and a[0].shape == (2, 3, 5, 4)
    c = fa_inputs.draw_f32((2, 3, 5, 4), seed=43, count=1)
    assert not np.array_equal(a[0], c[0])


def test_bf16_cast_is_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(20000).astype(np.float32)
    # add exact ties: values halfway between two bfloat16 neighbours
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    bits = fa_inputs.to_bf16_bits(x)
    val = oracle.decode_bf16(bits)
    up = oracle.decode_bf16(bits + np.uint16(1))
    dn = oracle.decode_bf16(bits - np.uint16(1))
    err = np.abs(x.astype(np.float64) - val)
    assert np.all(err <= np.abs(x - up)) and np.all(err <= np.abs(x - dn))
    is_tie = (err == np.abs(x - up)) | (err == np.abs(x - dn))
    assert is_tie.sum() >= 4000
    assert np.all(bits[is_tie] % 2 == 0)  # ties go to the even mantissa


def test_e4m3fn_quantiser():
    x = np.random.default_rng(1).standard_normal((3, 1000)).astype(np.float32)
    codes, s = fa_inputs.quantize_e4m3fn(x)
    assert s == np.float32(np.abs(x).max() / np.float32(448.0))
    grid = oracle.decode_e4m3fn(np.arange(256, dtype=np.uint8), 1.0)
    finite = np.sort(np.unique(grid[np.isfinite(grid)]))
    val = oracle.decode_e4m3fn(codes, 1.0)
    assert np.isfinite(val).all()
    y = (x / np.float32(s)).astype(np.float64)
    # nearest point of the e4m3fn grid
    idx = np.clip(np.searchsorted(finite, y), 1, finite.size - 1)
    nearest = np.minimum(np.abs(y - finite[idx - 1]), np.abs(y - finite[idx]))
    np.testing.assert_array_equal(np.abs(y - val), nearest)
    assert np.abs(val).max() == 448.0


def test_e4m3fn_saturates_and_handles_zero():
    codes, s = fa_inputs.quantize_e4m3fn(np.zeros(8, np.float32))
    assert s == 1.0 and np.all(oracle.decode_e4m3fn(codes) == 0.0)
    x = np.array([1.0, -1.0, 0.5, 1e-6], np.float32)
    codes, s = fa_inputs.quantize_e4m3fn(x)
    assert codes[0] == 0x7E and codes[1] == 0xFE  # +-448, the amax element
    assert oracle.decode_e4m3fn(codes[2:3])[0] == 224.0
    assert oracle.decode_e4m3fn(codes[3:4])[0] == 0.0  # 4.5e-4 rounds to zero (min 2^-9)


def test_make_inputs_formats():
    for dtype, npdt in (("fp32", np.float32), ("bf16", np.uint16), ("fp8", np.uint8)):
        inp = fa_inputs.make_inputs((1, 2, 7, 64), dtype, seed=3, with_dout=(dtype != "fp8"))
        assert inp.q.dtype == npdt and inp.q.shape == (1, 2, 7, 64)
        assert (inp.dout is None) == (dtype == "fp8")


def test_workload_table():
    w = fa_inputs.WORKLOADS
    assert len(w) == 5
    c3 = w["bf16_causal_fwd_b2h32n8192d128"]
    assert c3.shape == (2, 32, 8192, 128) and c3.causal and not c3.backward
    assert abs(c3.scale - 128 ** -0.5) < 1e-15
    assert w["fp32_fwdbwd_b1h1n128d64"].backward
    assert w["fp8_fwd_b1h32n16384d128"].dtype == "fp8"
