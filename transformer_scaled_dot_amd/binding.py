"""Python binding of the C ABI in include/attn_fwd.h and include/attn_bwd.h (argument
marshalling only).

`attn_fwd`, `attn_fwd_window`, `attn_decode`, `attn_decode_workspace_size`, `attn_decode_noalloc`,
`attn_bwd`, `attn_bwd_window`, `attn_bwd_workspace_size` and `attn_status_str` mirror the C entry points one
to one (raw device pointers, sizes, a stream handle).  `fwd`, `decode` and `bwd` are the tensor-level
conveniences: they check the tensors on the host, allocate the outputs (and workspaces) with
torch on the current stream and call the matching entry point; `attention` joins the forward
and the backward into one differentiable op for PyTorch code.  Every step of
the computation runs in the HIP kernels of libattn_fwd.so; if that library is missing this
module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_fwd.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
ATTN_OK = 0
STATUS = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_HEAD_DIM",
    -4: "ATTN_ERR_DTYPE", -5: "ATTN_ERR_SCALE", -6: "ATTN_ERR_LAUNCH", -7: "ATTN_ERR_FLAG",
    -8: "ATTN_ERR_ALIGN", -9: "ATTN_ERR_WINDOW", -10: "ATTN_ERR_WORKSPACE", -11: "ATTN_ERR_SCRATCH",
}
EXPORTS = ("attn_fwd", "attn_fwd_window", "attn_decode", "attn_decode_workspace_size", "attn_decode_noalloc",
           "attn_bwd", "attn_bwd_window", "attn_bwd_workspace_size", "attn_status_str")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"attention call failed: {STATUS.get(status, status)} ({attn_status_str(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn_fwd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m transformer_scaled_dot_amd.build`"
                           " (there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
    ]
    lib.attn_fwd_window.restype = ctypes.c_int
    lib.attn_fwd_window.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
    ]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p,
    ]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
    ]
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_workspace_size.argtypes = [ctypes.c_int] * 6
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p,
    ]
    lib.attn_bwd_window.restype = ctypes.c_int
    lib.attn_bwd_window.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p,
    ]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int] * 3
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens, dtype, stream) -> int:
    """The C entry point: device pointers as ints (or None), sizes, dtype code, stream handle."""
    return load_library().attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens,
                                   dtype, stream)


def attn_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window, key_lens, dtype,
                    stream) -> int:
    """The C entry point with a local band |i - j| <= window (-1: no band)."""
    return load_library().attn_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window,
                                          key_lens, dtype, stream)


def attn_decode(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens, dtype, workspace,
                workspace_bytes, stream) -> int:
    """The C entry point for queries at the end of a KV cache (key split + merge)."""
    return load_library().attn_decode(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens,
                                      dtype, workspace, workspace_bytes, stream)


def attn_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens, dtype, stream) -> int:
    """The C entry point of attn_decode with the library's static scratch (no workspace)."""
    return load_library().attn_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens,
                                              dtype, stream)


def attn_decode_workspace_size(B, H, Nq, Nk, D, dtype) -> int:
    return int(load_library().attn_decode_workspace_size(B, H, Nq, Nk, D, dtype))


def attn_bwd(q, k, v, o, dout, lse, dlse, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, key_lens,
             dtype, workspace, workspace_bytes, stream) -> int:
    """The C entry point of the backward (dQ, dK, dV from dO and the forward's O and LSE)."""
    return load_library().attn_bwd(q, k, v, o, dout, lse, dlse, dq, dk, dv, B, H, Nq, Nk, D, scale,
                                   causal, key_lens, dtype, workspace, workspace_bytes, stream)


def attn_bwd_window(q, k, v, o, dout, lse, dlse, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, window,
                    key_lens, dtype, workspace, workspace_bytes, stream) -> int:
    """The C entry point of the backward with a local band |i - j| <= window (-1: no band)."""
    return load_library().attn_bwd_window(q, k, v, o, dout, lse, dlse, dq, dk, dv, B, H, Nq, Nk, D,
                                          scale, causal, window, key_lens, dtype, workspace,
                                          workspace_bytes, stream)


def attn_bwd_workspace_size(B, H, Nq) -> int:
    return int(load_library().attn_bwd_workspace_size(B, H, Nq))


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def _torch():
    import torch

    return torch


def dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
    if t.dtype not in codes:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return codes[t.dtype]


def _check(q, k, v, key_lens, scale, out, lse, stream):
    """Host checks shared by fwd, decode and bwd; returns the marshalled arguments."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, D]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, D) or tuple(v.shape) != (B, H, Nk, D):
        raise ValueError(f"k and v must be [B={B}, H={H}, Nk, D={D}]; got {tuple(k.shape)}, {tuple(v.shape)}")
    if D not in (64, 128):
        raise ValueError(f"head dimension must be 64 or 128, got {D}")
    if min(B, H, Nq, Nk) < 1:
        raise ValueError("B, H, Nq and Nk must be >= 1")
    code = dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if not math.isfinite(scale):
        raise ValueError("scale must be finite")
    kl_ptr = None
    if key_lens is not None:
        if (not isinstance(key_lens, torch.Tensor) or key_lens.dtype != torch.int32
                or key_lens.device != q.device or tuple(key_lens.shape) != (B,)
                or not key_lens.is_contiguous()):
            raise ValueError("key_lens must be a contiguous int32 tensor [B] on q's device")
        kl_ptr = key_lens.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32 or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Nq]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return B, H, Nq, Nk, D, code, float(scale), kl_ptr, out, lse, handle


def decode(q, k, v, *, causal: bool = False, key_lens=None, scale: float | None = None, out=None,
           lse=None, workspace=None, stream=None):
    """O, LSE for Nq new queries that are the last Nq positions of each cached sequence.
    q: [B,H,Nq,D]; k, v: [B,H,Nk,D] (the cache, already holding the new tokens' keys and
    values); key_lens: int32 [B] valid cache lengths or None.  causal=True keeps, for query i,
    the keys j <= i + L_b - Nq.  workspace: a CUDA tensor of at least
    attn_decode_workspace_size(...) bytes, or None to allocate one with torch."""
    torch = _torch()
    B, H, Nq, Nk, D, code, scale, kl_ptr, out, lse, handle = _check(q, k, v, key_lens, scale, out,
                                                                  lse, stream)
    need = attn_decode_workspace_size(B, H, Nq, Nk, D, code)
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif not isinstance(workspace, torch.Tensor) or workspace.device != q.device \
                or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     B, H, Nq, Nk, D, scale, int(bool(causal)), kl_ptr, code, ws_ptr, ws_bytes,
                     handle)
    if rc != ATTN_OK:
        raise AttnError(rc)
    return out, lse


def fwd(q, k, v, *, causal: bool = False, key_lens=None, scale: float | None = None, out=None,
        lse=None, stream=None, window: int | None = None):
    """O, LSE = attention(q, k, v).  q: [B,H,Nq,D]; k, v: [B,H,Nk,D]; all contiguous CUDA tensors
    of one dtype; key_lens: int32 [B] on the same device or None.  scale defaults to 1/sqrt(D).
    window=w keeps only keys with |i - j| <= w (sliding-window attention); None: every key.
    Returns O (q's dtype, [B,H,Nq,D]) and LSE (float32, [B,H,Nq])."""
    if window is not None and (int(window) != window or window < 0):
        raise ValueError("window must be None or an integer >= 0")
    B, H, Nq, Nk, D, code, scale, kl_ptr, out, lse, handle = _check(q, k, v, key_lens, scale, out,
                                                                  lse, stream)
    if window is None:
        rc = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, Nq, Nk, D, scale, int(bool(causal)), kl_ptr, code, handle)
    else:
        rc = attn_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, Nq, Nk, D, scale, int(bool(causal)),
                             min(int(window), 2**31 - 1), kl_ptr, code, handle)
    if rc != ATTN_OK:
        raise AttnError(rc)
    return out, lse


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, key_lens=None, scale: float | None = None,
        dlse=None, dq=None, dk=None, dv=None, workspace=None, stream=None, window: int | None = None):
    """dQ, dK, dV of attention(q, k, v) for the gradient `dout` of O (and `dlse` of LSE, or None).
    o and lse are the forward's outputs for the same q, k, v, causal, key_lens, scale and window.
    Tensors as for fwd (fp32, bf16 or fp16); returns (dq, dk, dv) in q's dtype."""
    if window is not None and (int(window) != window or window < 0):
        raise ValueError("window must be None or an integer >= 0")
    torch = _torch()
    B, H, Nq, Nk, D, code, scale, kl_ptr, out, lse_t, handle = _check(q, k, v, key_lens, scale, o, lse,
                                                                       stream)
    if out is not o or lse_t is not lse:
        raise ValueError("o and lse must be the forward's outputs")
    if not isinstance(dout, torch.Tensor) or dout.shape != q.shape or dout.dtype != q.dtype \
            or dout.device != q.device or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous tensor like q")
    if dlse is not None and (not isinstance(dlse, torch.Tensor) or tuple(dlse.shape) != (B, H, Nq)
                             or dlse.dtype != torch.float32 or dlse.device != q.device
                             or not dlse.is_contiguous()):
        raise ValueError("dlse must be a contiguous float32 tensor [B, H, Nq] or None")
    outs = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
        elif t.shape != like.shape or t.dtype != like.dtype or t.device != like.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like its input")
        outs.append(t)
    need = attn_bwd_workspace_size(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
    rc = attn_bwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                         lse.data_ptr(), None if dlse is None else dlse.data_ptr(), outs[0].data_ptr(),
                         outs[1].data_ptr(), outs[2].data_ptr(), B, H, Nq, Nk, D, scale, int(bool(causal)),
                         -1 if window is None else min(int(window), 2**31 - 1), kl_ptr, code,
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(), handle)
    if rc != ATTN_OK:
        raise AttnError(rc)
    return tuple(outs)


def _attention_function():
    """The torch.autograd.Function behind `attention` (built on first use: importing this module
    does not import torch)."""
    global _AttentionFn
    if _AttentionFn is not None:
        return _AttentionFn
    torch = _torch()

    class AttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, key_lens, window):
            o, lse = fwd(q, k, v, causal=causal, key_lens=key_lens, scale=scale, window=window)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.key_lens, ctx.causal, ctx.scale, ctx.window = key_lens, causal, scale, window
            ctx.set_materialize_grads(False)  # an unused output's gradient arrives as None
            return o, lse

        @staticmethod
        def backward(ctx, do, dlse):
            q, k, v, o, lse = ctx.saved_tensors
            if do is None:  # only the LSE reaches the loss
                do = torch.zeros_like(o)
            dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, key_lens=ctx.key_lens,
                             scale=ctx.scale, dlse=None if dlse is None else dlse.contiguous(),
                             window=ctx.window)
            return dq, dk, dv, None, None, None, None

    _AttentionFn = AttentionFn
    return AttentionFn


_AttentionFn = None


def attention(q, k, v, *, causal: bool = False, scale: float | None = None, key_lens=None,
              window: int | None = None, return_lse: bool = False):
    """Differentiable attention for PyTorch code: O = softmax(scale q k^T + mask) v per (b, h),
    with the forward and backward of this library (attn_fwd_window / attn_bwd_window) as the
    two passes.  Tensors as for `fwd` ([B, H, N, D], contiguous, CUDA, fp32 / fp16 / bf16);
    key_lens (int32 [B]) and window as for `fwd`.  Returns O, or (O, LSE) with return_lse=True,
    in which case a loss may also depend on LSE (its gradient enters the backward as dLSE)."""
    o, lse = _attention_function().apply(q, k, v, bool(causal), scale, key_lens, window)
    return (o, lse) if return_lse else o
