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


# --------------------------------------------------------------------------- #
# Microscaled fp8 (e8m0 scale per 32 consecutive elements)
# --------------------------------------------------------------------------- #
def test_mx_scale_byte_closed_form():
    # one block per row: the scale byte is floor(log2 amax) - 8 + 127
    rows = [(1.0, 119), (448.0, 127), (3.0, 120), (0.75, 118), (2.0 ** 10, 129), (0.0, 0)]
    x = np.zeros((len(rows), 32), np.float32)
    for i, (amax, _) in enumerate(rows):
        x[i, 5] = -amax
    _, e = fa_inputs.quantize_mx_e4m3fn(x, -1)
    assert e.shape == (len(rows), 1)
    assert [int(v) for v in e[:, 0]] == [b for _, b in rows]
    # and the decoder reads byte E as 2^(E - 127)
    one = np.full((1, 32), 0x38, np.uint8)  # e4m3fn code of 1.0
    for byte, value in ((127, 1.0), (128, 2.0), (120, 2.0 ** -7), (0, 2.0 ** -127)):
        got = oracle.decode_mx_e4m3fn(one, np.array([[byte]], np.uint8), -1)
        assert np.all(got == value)


def test_mx_roundtrip_is_exact_on_representable_blocks():
    # blocks of (small integer m) * 2^k with |m| <= 14 and amax 14 * 2^k: the
    # scale is 2^(k - 5), every element is m * 32 <= 448 with at most four
    # significant bits -- an e4m3 value -- so nothing rounds
    rng = np.random.default_rng(5)
    k = rng.integers(-20, 20, size=(6, 4, 1))
    m = rng.integers(-14, 15, size=(6, 4, 32)).astype(np.float64)
    m[..., 0] = 14.0
    x = (m * np.exp2(k)).reshape(6, 128).astype(np.float32)
    codes, e = fa_inputs.quantize_mx_e4m3fn(x, -1)
    np.testing.assert_array_equal(oracle.decode_mx_e4m3fn(codes, e, -1), x.astype(np.float64))


def test_mx_blocks_follow_the_axis():
    # V is blocked along the sequence axis: changing one element moves only
    # the scale of its own 32-row block of that column
    x = np.ones((1, 1, 70, 8), np.float32)
    _, e0 = fa_inputs.quantize_mx_e4m3fn(x, -2)
    assert e0.shape == (1, 1, 3, 8)
    x[0, 0, 40, 3] = 1000.0
    _, e1 = fa_inputs.quantize_mx_e4m3fn(x, -2)
    changed = np.argwhere(e1 != e0)
    assert changed.tolist() == [[0, 0, 1, 3]]


def test_mx_error_is_within_the_format_step():
    x = np.random.default_rng(2).standard_normal((4, 256)).astype(np.float32)
    x *= np.exp2(np.random.default_rng(3).uniform(-6, 6, size=(4, 1))).astype(np.float32)
    codes, e = fa_inputs.quantize_mx_e4m3fn(x, -1)
    y = oracle.decode_mx_e4m3fn(codes, e, -1)
    scale = np.repeat(np.exp2(e.astype(np.float64) - 127), 32, axis=-1)
    # e4m3 normal numbers carry 3 mantissa bits: RNE error <= 2^-4 relative;
    # below 2^-6 (subnormal) the step is 2^-9, absolute, in units of the
    # scale; and x / scale can reach up to 512, above the largest code 448,
    # where the quantiser saturates (the OCP choice of the shared exponent)
    bound = np.maximum.reduce([np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10,
                               np.abs(x) - 448.0 * scale])
    assert np.all(np.abs(y) <= 448.0 * scale)
    assert np.all(np.abs(y - x) <= bound)


def test_make_mx_inputs_layout():
    mx = fa_inputs.make_mx_inputs((1, 2, 70, 64), seed=3)
    assert mx.q.shape == (1, 2, 70, 64) and mx.q.dtype == np.uint8
    assert mx.qs.shape == mx.ks.shape == (1, 2, 70, 4) and mx.vs.shape == (1, 2, 3, 64)
    assert np.all(mx.qs[..., 2:] == 127)
