"""The C-ABI library: it loads, exports what include/fa.h declares, and rejects
bad arguments before launching anything (no GPU needed: every call here fails
validation or has no work, so no HIP call is made)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "fa_probe.h")

fa = pytest.importorskip("exact_io_aware_11_amd")
lib = fa.lib

OK, INVALID, UNSUPPORTED = fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
P = 0x10000  # a 16-byte aligned fake address; never dereferenced in these tests


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_bias", "fa_bwd_delta", "fa_bwd_dkdv",
                                    "fa_bwd_dq", "fa_bwd_noalloc", "fa_bwd_workspace_size",
                                    "fa_fwd", "fa_fwd_bias", "fa_fwd_mxfp8",
                                    "fa_status_string", "fa_std_fwd", "fa_std_workspace_size"]
    assert declared_functions(PROBE_HEADER) == ["fa_measure_mfma_rate"]


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(fa._lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(fa._lib.SIGNATURES) == set(declared_functions())
    # the rate probe lives in its own library, not in the attention one
    assert not hasattr(raw, "fa_measure_mfma_rate")
    probe = ctypes.CDLL(fa.probe.PROBE_LIB_PATH)
    for name in declared_functions(PROBE_HEADER):
        assert hasattr(probe, name), name
    assert set(fa.probe.SIGNATURES) == set(declared_functions(PROBE_HEADER))


def test_probe_status_codes_match_the_attention_ones():
    """fa_probe.h repeats fa.h's element-type and status values."""
    def enum_values(header):
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        return {k: int(v) for k, v in re.findall(r"\b(FA_[A-Z0-9_]+)\s*=\s*(\d+)", text)}
    main, probe = enum_values(HEADER), enum_values(PROBE_HEADER)
    for name in ("FP32", "BF16", "FP8_E4M3", "OK", "ERR_INVALID_ARG", "ERR_UNSUPPORTED", "ERR_HIP"):
        assert probe["FA_PROBE_" + name] == main["FA_" + name], name


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, scale=0.125, causal=0,
             dtype=fa.FA_BF16, qd=1.0, kd=1.0, vd=1.0, stream=None)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                      a["scale"], a["causal"], a["dtype"], a["qd"], a["kd"], a["vd"], a["stream"])


def fwd_mx(**kw):
    a = dict(q=P, k=P, v=P, qs=P, ks=P, vs=P, o=P, lse=P, B=1, H=1, N=16, d=64, scale=0.125,
             causal=0, stream=None)
    a.update(kw)
    return lib.fa_fwd_mxfp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"],
                            a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(d=0), INVALID), (dict(causal=3), INVALID),
    (dict(N=-1), INVALID), (dict(scale=0.0), INVALID), (dict(scale=math.nan), INVALID),
    (dict(qs=0), INVALID), (dict(ks=0), INVALID), (dict(vs=0), INVALID), (dict(q=0), INVALID),
    (dict(qs=P + 1), INVALID), (dict(vs=P + 2), INVALID), (dict(v=P + 4), INVALID),
])
def test_fwd_mxfp8_rejects_before_launch(kw, status):
    assert fwd_mx(**kw) == status


def test_fwd_mxfp8_empty_is_a_noop():
    assert fwd_mx(N=0, qs=0, ks=0, vs=0) == OK and fwd_mx(B=0) == OK


def fwd_b(**kw):
    a = dict(q=P, k=P, v=P, bias=P, sb=0, sh=0, sq=16, o=P, lse=P, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return lib.fa_fwd_bias(a["q"], a["k"], a["v"], a["bias"], a["sb"], a["sh"], a["sq"], a["o"],
                           a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                           a["dtype"], a["stream"])


def bwd_b(**kw):
    a = dict(q=P, k=P, v=P, bias=P, sb=0, sh=0, sq=16, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P,
             wsb=1 << 20, B=1, H=1, N=16, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return lib.fa_bwd_bias(a["q"], a["k"], a["v"], a["bias"], a["sb"], a["sh"], a["sq"], a["o"],
                           a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], a["B"],
                           a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                           a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_FP8_E4M3), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(bias=P + 4), INVALID), (dict(sq=18), INVALID), (dict(sb=-4), INVALID),
    (dict(sh=2), INVALID), (dict(sq=1 << 30), INVALID), (dict(N=1 << 16, sq=1 << 16), INVALID),
    (dict(q=0), INVALID), (dict(scale=0.0), INVALID), (dict(causal=2), INVALID),
])
@pytest.mark.parametrize("fn", [fwd_b, bwd_b])
def test_bias_entry_points_reject_before_launch(kw, status, fn):
    assert fn(**kw) == status


def test_bias_entry_points_empty_is_a_noop():
    assert fwd_b(N=0) == OK and fwd_b(B=0, bias=0) == OK and bwd_b(H=0) == OK


def bwd(fn="fa_bwd", **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, wsb=1 << 20, B=1, H=1,
             N=16, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                      a["dv"], a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                      a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(d=0), INVALID),
    (dict(d=-64), INVALID), (dict(dtype=3), INVALID), (dict(dtype=-1), INVALID),
    (dict(causal=2), INVALID), (dict(B=-1), INVALID), (dict(H=-2), INVALID),
    (dict(N=-1), INVALID), (dict(scale=0.0), INVALID), (dict(scale=-0.1), INVALID),
    (dict(scale=math.nan), INVALID), (dict(scale=math.inf), INVALID),
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID), (dict(o=0), INVALID),
    (dict(lse=0), INVALID), (dict(q=P + 8), INVALID), (dict(o=P + 2), INVALID),
    (dict(lse=P + 2), INVALID),
    (dict(dtype=fa.FA_FP8_E4M3, qd=0.0), INVALID),
    (dict(dtype=fa.FA_FP8_E4M3, vd=math.nan), INVALID),
    (dict(B=1 << 20, H=1 << 20, N=1 << 20), INVALID),
])
def test_fwd_rejects_before_launch(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=0, k=0, v=0)])
def test_fwd_empty_is_a_noop(kw):
    assert fwd(**kw) == OK


@pytest.mark.parametrize("name,status", [("", OK), ("interleaved", OK), ("pingpong", OK),
                                         ("rows64", OK), ("ping-pong", INVALID), ("w64", INVALID)])
def test_fwd_schedule_names(monkeypatch, name, status):
    """FA_FWD_SCHEDULE is read on every forward call and an unknown name is
    rejected before any launch (an empty problem launches nothing anyway)."""
    monkeypatch.setenv("FA_FWD_SCHEDULE", name)
    assert fwd(B=0) == status
    assert fwd_b(B=0) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_FP8_E4M3), UNSUPPORTED), (dict(d=80), UNSUPPORTED),
    (dict(dtype=9), INVALID), (dict(causal=-1), INVALID), (dict(scale=0.0), INVALID),
    (dict(ws=0), INVALID), (dict(do=0), INVALID), (dict(dq=0), INVALID),
    (dict(dk=P + 4), INVALID), (dict(ws=P + 2), INVALID), (dict(wsb=16), INVALID),
])
@pytest.mark.parametrize("fn", ["fa_bwd", "fa_bwd_delta", "fa_bwd_dkdv", "fa_bwd_dq"])
def test_bwd_rejects_before_launch(kw, status, fn):
    assert bwd(fn, **kw) == status


def test_bwd_empty_is_a_noop():
    assert bwd(N=0) == OK and bwd(B=0, q=0) == OK


def bwd_noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                              a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_FP8_E4M3), UNSUPPORTED), (dict(d=80), UNSUPPORTED),
    (dict(dtype=9), INVALID), (dict(causal=-1), INVALID), (dict(scale=0.0), INVALID),
    (dict(do=0), INVALID), (dict(dq=0), INVALID), (dict(dk=P + 4), INVALID),
    (dict(lse=P + 2), INVALID), (dict(B=-1), INVALID),
    # beyond the scratch: one row too many, in several splits of B * H * N
    (dict(N=fa.FA_NOALLOC_MAX_ROWS + 1), UNSUPPORTED),
    (dict(B=2, H=8, N=fa.FA_NOALLOC_MAX_ROWS // 16 + 1), UNSUPPORTED),
    (dict(B=1 << 11, H=1 << 11, N=2), UNSUPPORTED),
])
def test_bwd_noalloc_rejects_before_launch(kw, status):
    assert bwd_noalloc(**kw) == status


def test_bwd_noalloc_empty_is_a_noop():
    assert bwd_noalloc(N=0) == OK and bwd_noalloc(B=0, q=0) == OK


@pytest.mark.parametrize("args,status", [
    ((0, 256, 10, 1), INVALID), ((P + 2, 256, 10, 1), INVALID), ((P, 0, 10, 1), INVALID),
    ((P, 65537, 10, 1), INVALID), ((P, 256, 0, 2), INVALID), ((P, 256, 1 << 21, 1), INVALID),
    ((P, 256, 10, 0), UNSUPPORTED), ((P, 256, 10, 7), INVALID)])
def test_rate_probe_rejects_before_launch(args, status):
    assert fa.probe.probe_lib.fa_measure_mfma_rate(*args, None) == status


def std(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, ws=P, wsb=1 << 30, B=1, H=1, N=16, d=64, scale=0.125,
             causal=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return lib.fa_std_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["wsb"], a["B"],
                          a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                          a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_FP32), UNSUPPORTED), (dict(dtype=fa.FA_FP8_E4M3), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED), (dict(dtype=7), INVALID), (dict(causal=2), INVALID),
    (dict(scale=0.0), INVALID), (dict(q=0), INVALID), (dict(ws=0), INVALID),
    (dict(ws=P + 16), INVALID), (dict(o=P + 4), INVALID), (dict(wsb=100), INVALID),
    (dict(B=1 << 9, H=1 << 8, wsb=1 << 62), UNSUPPORTED),
])
def test_std_rejects_before_launch(kw, status):
    assert std(**kw) == status


def test_std_workspace_size():
    # S float32 and P bf16, rows padded to 64 entries, each part 256-byte rounded
    assert lib.fa_std_workspace_size(1, 1, 16, 64) == 16 * 64 * 4 + 2048
    assert lib.fa_std_workspace_size(2, 3, 100, 128) == 6 * 100 * 128 * 4 + 6 * 100 * 128 * 2
    assert lib.fa_std_workspace_size(1, 1, 3, 96) == 0
    assert std(N=0) == OK and std(B=0, ws=0) == OK


def test_workspace_size():
    assert lib.fa_bwd_workspace_size(2, 16, 4096, 128) == 2 * 16 * 4096 * 4
    assert lib.fa_bwd_workspace_size(1, 1, 3, 64) == 256  # rounded up to 256 bytes
    assert lib.fa_bwd_workspace_size(1, 1, 3, 96) == 0
    assert lib.fa_bwd_workspace_size(-1, 1, 3, 64) == 0
    assert fa.fa_bwd_workspace_size(2, 16, 4096, 128) == 2 * 16 * 4096 * 4


def test_status_strings():
    for s in (0, 1, 2, 3, 99, -5):
        assert isinstance(fa.fa_status_string(s), str) and fa.fa_status_string(s)
    assert fa.fa_status_string(OK) == "ok"


def test_flop_counts():
    assert fa.flops_fwd(2, 32, 8192, 128, True) == 2 * 2 * 32 * 8192 ** 2 * 128
    assert fa.flops_bwd(2, 16, 4096, 128, True) == 5 * 2 * 16 * 4096 ** 2 * 128
