"""Argument marshalling from torch tensors to the C ABI (include/fa.h)."""
from __future__ import annotations

from ._lib import FA_BF16, FA_FP8_E4M3, FA_FP32, FA_OK, FAError, lib


def dtype_code(t) -> int:
    """fa_dtype of a tensor: float32, bfloat16, or e4m3fn codes (float8_e4m3fn or uint8)."""
    import torch

    if t.dtype == torch.float32:
        return FA_FP32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _stream_handle(stream) -> int:
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(int(x) for x in q.shape)


def _check_device(name, t):
    """The kernels dereference the pointers on the GPU: host tensors must not
    reach them."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")


def _check_like(name, t, shape):
    _check_device(name, t)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_dtypes(code, inputs, outputs):
    """The C ABI sees only pointers: make sure every buffer has the element
    type (and so the byte size) the kernels will assume for `code`."""
    import torch

    for name, t in inputs:
        if dtype_code(t) != code:
            raise TypeError(f"{name} has dtype {t.dtype}, inconsistent with the other inputs")
    want = torch.float32 if code == FA_FP32 else torch.bfloat16
    for name, t in outputs:
        if t.dtype != want:
            raise TypeError(f"{name} must be {want}, got {t.dtype}")


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, descale=(1.0, 1.0, 1.0), stream=None):
    """Enqueue the forward pass.  Writes o ([B,H,N,d]) and lse ([B,H,N] float32)."""
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    code = dtype_code(q)
    _check_dtypes(code, (("k", k), ("v", v)), (("o", o),))
    if lse.dtype != __import__("torch").float32:
        raise TypeError("lse must be float32")
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, N, d, float(scale), int(bool(causal)), dtype_code(q),
                    float(descale[0]), float(descale[1]), float(descale[2]),
                    _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd: " + fa_status_string(st))


def fa_fwd_mxfp8(q, k, v, q_scale, k_scale, v_scale, o, lse, scale: float, causal: bool,
                 stream=None):
    """Enqueue the forward pass on fp8 e4m3fn codes with e8m0 block scales:
    q_scale, k_scale [B,H,N,4] (bytes 0 .. d/32-1 of each row used) and
    v_scale [B,H,ceil(N/32),d] (uint8).
    Writes o ([B,H,N,d] bfloat16) and lse ([B,H,N] float32)."""
    import torch

    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    _check_dtypes(FA_FP8_E4M3, (("q", q), ("k", k), ("v", v)), (("o", o),))
    if d % 32:
        raise ValueError("d must be a multiple of 32")
    for name, t, shape in (("q_scale", q_scale, (B, H, N, 4)),
                           ("k_scale", k_scale, (B, H, N, 4)),
                           ("v_scale", v_scale, (B, H, (N + 31) // 32, d))):
        _check_like(name, t, shape)
        if t.dtype != torch.uint8:
            raise TypeError(f"{name} must be uint8 (e8m0 exponents)")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    st = lib.fa_fwd_mxfp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(),
                          k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, N, d, float(scale), int(bool(causal)), _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_mxfp8: " + fa_status_string(st))


def _bias_view(bias, B, H, N):
    """A float32 bias tensor broadcast to [B, H, N, N]: (pointer, strides b, h, q)."""
    import torch

    _check_device("bias", bias)
    if bias.dtype != torch.float32:
        raise TypeError("bias must be float32")
    if bias.dim() != 4:
        raise ValueError("bias must be 4-D, broadcastable to [B, H, N, N]")
    b = bias.expand(B, H, N, N)
    if b.stride(3) != 1:
        raise ValueError("bias must have unit stride along the key dimension")
    return b.data_ptr(), b.stride(0), b.stride(1), b.stride(2)


def fa_fwd_bias(q, k, v, bias, o, lse, scale: float, causal: bool, stream=None):
    """Enqueue the forward pass with an additive float32 bias on the scaled
    scores (-inf masks a key).  bias is a 4-D tensor broadcastable to
    [B, H, N, N] whose strides (in elements) are multiples of 4 and whose last
    stride is 1 (a view of a row-pitched buffer works).  Writes o and lse;
    rows with no finite score get o = 0 and lse = -inf."""
    import torch

    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    code = dtype_code(q)
    if code == FA_FP8_E4M3:
        raise FAError(2, "fa_fwd_bias: float32 or bfloat16 inputs")
    _check_dtypes(code, (("k", k), ("v", v)), (("o", o),))
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    bp, sb, sh, sq = _bias_view(bias, B, H, N)
    st = lib.fa_fwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), bp, sb, sh, sq, o.data_ptr(),
                         lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), code,
                         _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_bias: " + fa_status_string(st))


def fa_bwd_bias(q, k, v, bias, o, dout, lse, dq, dk, dv, workspace, scale: float, causal: bool,
                stream=None):
    """Enqueue the backward pass with the bias of fa_fwd_bias (an input: no
    gradient is formed for it).  Writes dq, dk, dv."""
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    code = dtype_code(q)
    if code == FA_FP8_E4M3:
        raise FAError(2, "fa_bwd_bias: the backward takes float32 or bfloat16 tensors")
    _check_dtypes(code, (("k", k), ("v", v), ("o", o), ("dout", dout)),
                  (("dq", dq), ("dk", dk), ("dv", dv)))
    bp, sb, sh, sq = _bias_view(bias, B, H, N)
    _check_device("workspace", workspace)
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.fa_bwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), bp, sb, sh, sq, o.data_ptr(),
                         dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                         dv.data_ptr(), workspace.data_ptr(), nbytes, B, H, N, d, float(scale),
                         int(bool(causal)), code, _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_bias: " + fa_status_string(st))


def fa_std_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(lib.fa_std_workspace_size(B, H, N, d))


def fa_std_fwd(q, k, v, o, lse, workspace, scale: float, causal: bool, stream=None):
    """Enqueue standard attention with S and P written to the workspace (uint8
    device tensor of fa_std_workspace_size bytes, 256-byte aligned): the
    materialising baseline of the IO comparison.  bf16 only; writes o, lse."""
    import torch

    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    code = dtype_code(q)
    _check_dtypes(code, (("k", k), ("v", v)), (("o", o),))
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check_device("workspace", workspace)
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.fa_std_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        workspace.data_ptr(), nbytes, B, H, N, d, float(scale),
                        int(bool(causal)), code, _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_std_fwd: " + fa_status_string(st))


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(lib.fa_bwd_workspace_size(B, H, N, d))


def _bwd_call(fn_name, q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, stream):
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    code = dtype_code(q)
    if code == FA_FP8_E4M3:
        raise FAError(2, f"{fn_name}: the backward takes float32 or bfloat16 tensors")
    _check_dtypes(code, (("k", k), ("v", v), ("o", o), ("dout", dout)),
                  (("dq", dq), ("dk", dk), ("dv", dv)))
    _check_device("workspace", workspace)
    nbytes = workspace.numel() * workspace.element_size()
    st = getattr(lib, fn_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), workspace.data_ptr(), nbytes, B, H, N, d,
                               float(scale), int(bool(causal)), dtype_code(q),
                               _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, f"{fn_name}: " + fa_status_string(st))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale: float, causal: bool,
           stream=None):
    """Enqueue the backward pass.  Writes dq, dk, dv; workspace (uint8 device
    tensor of fa_bwd_workspace_size bytes) receives delta in its first B*H*N floats."""
    _bwd_call("fa_bwd", q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, stream)


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool, stream=None):
    """fa_bwd without a workspace: delta lives in the library's per-GPU scratch
    (B*H*N <= FA_NOALLOC_MAX_ROWS; calls that overlap on one GPU race on it).
    Writes dq, dk, dv, bitwise as fa_bwd does."""
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_like(name, t, (B, H, N, d))
    _check_like("lse", lse, (B, H, N))
    code = dtype_code(q)
    if code == FA_FP8_E4M3:
        raise FAError(2, "fa_bwd_noalloc: the backward takes float32 or bfloat16 tensors")
    _check_dtypes(code, (("k", k), ("v", v), ("o", o), ("dout", dout)),
                  (("dq", dq), ("dk", dk), ("dv", dv)))
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), code,
                            _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_noalloc: " + fa_status_string(st))


def fa_bwd_delta(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, stream=None):
    """Backward stage: delta into the workspace (fa_bwd runs it for float32;
    for bf16 the dQ stage forms delta itself)."""
    _bwd_call("fa_bwd_delta", q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal,
              stream)


def fa_bwd_dkdv(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, stream=None):
    """Backward stage: dK and dV, reading delta from the workspace."""
    _bwd_call("fa_bwd_dkdv", q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal,
              stream)


def fa_bwd_dq(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, stream=None):
    """Backward stage: dQ (bf16: also writes delta to the workspace; float32:
    reads it).  fa_bwd is fa_bwd_dq then fa_bwd_dkdv for bf16, and
    fa_bwd_delta, fa_bwd_dkdv, fa_bwd_dq for float32."""
    _bwd_call("fa_bwd_dq", q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, stream)


def fa_status_string(status: int) -> str:
    return lib.fa_status_string(int(status)).decode()


def flops_fwd(B, H, N, d, causal) -> float:
    """Algorithmic forward FLOPs: 4 B H N^2 d, halved under the causal mask."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def flops_bwd(B, H, N, d, causal) -> float:
    """Algorithmic backward FLOPs: the five N x N x d products (S recompute, dV,
    dP, dQ, dK), 10 B H N^2 d, halved under the causal mask."""
    f = 10.0 * B * H * N * N * d
    return f / 2 if causal else f


__all__ = ["FA_FP32", "FA_BF16", "FA_FP8_E4M3", "dtype_code", "fa_fwd", "fa_fwd_bias",
           "fa_fwd_mxfp8", "fa_bwd", "fa_bwd_bias",
           "fa_bwd_delta", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_noalloc",
           "fa_bwd_workspace_size", "fa_std_fwd", "fa_std_workspace_size", "fa_status_string",
           "flops_fwd", "flops_bwd"]
