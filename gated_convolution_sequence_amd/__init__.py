"""MI355X (gfx950) Hyena-SE / Hyena-MR forward: y = q (.) (h * (k (.) v)).

A thin Python binding of the C ABI in ``include/hyena_conv.h``.  It only
checks and marshals arguments (device pointers, sizes, the current HIP
stream); every step of the computation runs in the HIP kernels of
``libhyena_conv.so``.  There is no fallback: if the library is missing or
rejects a call, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhyena_conv.so")

BLOCK_LEN = 64
SLAB = 128  # channels per 8-wave workgroup of the grouped forward (the 16-wave form takes 256)
WIDE_SLAB = 256
DTYPE_BF16 = 0
DTYPE_F32 = 1

STATUS = {
    0: "HYENA_OK", -1: "HYENA_ERR_NULL", -2: "HYENA_ERR_SHAPE", -3: "HYENA_ERR_GROUP",
    -4: "HYENA_ERR_FILTER_LEN", -5: "HYENA_ERR_ALIGN", -6: "HYENA_ERR_ALIAS",
    -7: "HYENA_ERR_UNSUPPORTED", -8: "HYENA_ERR_LAUNCH", -9: "HYENA_ERR_DTYPE",
    -10: "HYENA_ERR_WORKSPACE", -11: "HYENA_ERR_SCRATCH",
}

# Every symbol include/hyena_conv.h declares.
EXPORTS = ("hyena_conv_fwd", "hyena_conv_fwd_f32", "hyena_conv_fwd_ex", "hyena_conv_fwd_halo",
           "hyena_conv_bwd", "hyena_conv_bwd_workspace", "hyena_conv_fwd_long",
           "hyena_conv_fwd_long_workspace", "hyena_conv_plan", "hyena_conv_strerror",
           "hyena_conv_block_len", "hyena_conv_bwd_noalloc", "hyena_conv_scratch_bytes",
           "hyena_conv_fwd_long_ex", "hyena_conv_bwd_long", "hyena_conv_bwd_long_workspace",
           "hyena_conv_bwd_long_ex")


class HyenaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, strerror(status), STATUS.get(status, status)))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libhyena_conv.so is not built (expected at %s); run "
                "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        fwd_args = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp]
        for name in ("hyena_conv_fwd", "hyena_conv_fwd_f32"):
            fn = getattr(L, name)
            fn.argtypes = fwd_args
            fn.restype = ctypes.c_int
        L.hyena_conv_fwd_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp,
                                        ctypes.c_int, i64, vp]
        L.hyena_conv_fwd_ex.restype = ctypes.c_int
        L.hyena_conv_fwd_halo.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                          vp, ctypes.c_int, i64, vp]
        L.hyena_conv_fwd_halo.restype = ctypes.c_int
        L.hyena_conv_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                     vp, i64, ctypes.c_int, vp]
        L.hyena_conv_bwd.restype = ctypes.c_int
        L.hyena_conv_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                             vp, ctypes.c_int, vp]
        L.hyena_conv_bwd_noalloc.restype = ctypes.c_int
        L.hyena_conv_scratch_bytes.argtypes = []
        L.hyena_conv_scratch_bytes.restype = i64
        L.hyena_conv_bwd_workspace.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                               ctypes.POINTER(i64)]
        L.hyena_conv_bwd_workspace.restype = ctypes.c_int
        L.hyena_conv_fwd_long.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, ctypes.c_int,
                                          vp, i64, vp]
        L.hyena_conv_fwd_long.restype = ctypes.c_int
        L.hyena_conv_fwd_long_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, ctypes.c_int,
                                             vp, i64, ctypes.c_int, vp]
        L.hyena_conv_fwd_long_ex.restype = ctypes.c_int
        L.hyena_conv_fwd_long_workspace.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                                    ctypes.POINTER(i64)]
        L.hyena_conv_fwd_long_workspace.restype = ctypes.c_int
        L.hyena_conv_bwd_long.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                          ctypes.c_int, vp, i64, vp]
        L.hyena_conv_bwd_long.restype = ctypes.c_int
        L.hyena_conv_bwd_long_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                             ctypes.c_int, vp, i64, ctypes.c_int, vp]
        L.hyena_conv_bwd_long_ex.restype = ctypes.c_int
        L.hyena_conv_bwd_long_workspace.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                                    ctypes.POINTER(i64)]
        L.hyena_conv_bwd_long_workspace.restype = ctypes.c_int
        L.hyena_conv_plan.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64,
                                      ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.hyena_conv_plan.restype = ctypes.c_int
        L.hyena_conv_strerror.argtypes = [ctypes.c_int]
        L.hyena_conv_strerror.restype = ctypes.c_char_p
        L.hyena_conv_block_len.argtypes = []
        L.hyena_conv_block_len.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().hyena_conv_strerror(int(status)).decode()


def plan(B: int, L: int, D: int, group_size: int, l_h: int, dtype: int = DTYPE_BF16,
         span_chunks: int = 0):
    """(chunks per workgroup, workgroup count) the library would launch."""
    span = ctypes.c_int64()
    wgs = ctypes.c_int64()
    st = lib().hyena_conv_plan(B, L, D, group_size, l_h, dtype, span_chunks,
                               ctypes.byref(span), ctypes.byref(wgs))
    if st != 0:
        raise HyenaError(st, "hyena_conv_plan")
    return span.value, wgs.value


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return DTYPE_BF16
    if t == torch.float32:
        return DTYPE_F32
    raise TypeError("q, k, v, h must be bfloat16 or float32, got %s" % t)


def conv_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, h: torch.Tensor,
             group_size: int, out: Optional[torch.Tensor] = None, span_chunks: int = 0,
             stream: Optional[torch.cuda.Stream] = None, k_prev: Optional[torch.Tensor] = None,
             v_prev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = q (.) (h * (k (.) v)) on the GPU, enqueued on ``stream`` (default: current).

    q, k, v: [B, L, D] contiguous device tensors (bf16 or fp32, all alike);
    h: [D // group_size, l_h] of the same dtype.  Returns ``out`` ([B, L, D]).
    k_prev, v_prev ([B, P, D]): the rows that precede row 0 (a shard of a
    longer sequence); without them the history before row 0 is zero.
    """
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("h", h)):
        if t.dtype != dt:
            raise TypeError("%s has dtype %s, q has %s" % (name, t.dtype, dt))
        if t.device != dev or dev.type != "cuda":
            raise ValueError("%s must be a tensor on q's GPU" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    code = _dtype_code(dt)
    shape = q.shape
    if len(shape) != 3 or k.shape != shape or v.shape != shape:
        raise ValueError("q, k, v must share one [B, L, D] shape")
    if h.dim() != 2:
        raise ValueError("h must be [D // group_size, l_h]")
    B, L, D = shape
    G, l_h = h.shape
    if group_size < 1 or D % group_size != 0 or G != D // group_size:
        raise ValueError("h has %d filters; D=%d, group_size=%d" % (G, D, group_size))
    P = 0
    if (k_prev is None) != (v_prev is None):
        raise ValueError("pass both k_prev and v_prev, or neither")
    if k_prev is not None:
        for name, t in (("k_prev", k_prev), ("v_prev", v_prev)):
            if t.dtype != dt or t.device != dev or not t.is_contiguous():
                raise ValueError("%s must be a contiguous tensor like q" % name)
            if t.dim() != 3 or t.shape[0] != B or t.shape[2] != D or t.shape != k_prev.shape:
                raise ValueError("%s must be [B, P, D]" % name)
        P = k_prev.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != shape or out.dtype != dt or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if P == 0:
        fn = lib().hyena_conv_fwd_ex
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), B, L, D, group_size, l_h,
                out.data_ptr(), code, span_chunks, stream.cuda_stream)
    else:
        fn = lib().hyena_conv_fwd_halo
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), k_prev.data_ptr(),
                v_prev.data_ptr(), P, B, L, D, group_size, l_h, out.data_ptr(), code,
                span_chunks, stream.cuda_stream)
    if dev.index == torch.cuda.current_device():
        st = fn(*args)
    else:
        with torch.cuda.device(dev):
            st = fn(*args)
    if st != 0:
        raise HyenaError(st, fn.__name__)
    return out


def bwd_workspace_bytes(B: int, L: int, D: int, group_size: int, l_h: int,
                        dtype: int = DTYPE_BF16) -> int:
    """Workspace bytes hyena_conv_bwd needs for the filter gradient."""
    n = ctypes.c_int64()
    st = lib().hyena_conv_bwd_workspace(B, L, D, group_size, l_h, dtype, ctypes.byref(n))
    if st != 0:
        raise HyenaError(st, "hyena_conv_bwd_workspace")
    return n.value


def conv_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, h: torch.Tensor,
             dy: torch.Tensor, group_size: int, need_dq: bool = True, need_dkv: bool = True,
             need_dh: bool = True, stream: Optional[torch.cuda.Stream] = None):
    """Gradients (dq, dk, dv, dh) of y = q (.) (h * (k (.) v)) for upstream dy.

    dq, dk, dv have q's dtype; dh is float32 [D // group_size, l_h].  Parts
    not requested are returned as None.
    """
    dt, dev = q.dtype, q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("h", h), ("dy", dy)):
        if t.dtype != dt or t.device != dev or dev.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor like q" % name)
    if q.dim() != 3 or any(t.shape != q.shape for t in (k, v, dy)) or h.dim() != 2:
        raise ValueError("q, k, v, dy must be [B, L, D]; h [D // group_size, l_h]")
    code = _dtype_code(dt)
    B, L, D = q.shape
    G, l_h = h.shape
    if group_size < 1 or D % group_size != 0 or G != D // group_size:
        raise ValueError("h has %d filters; D=%d, group_size=%d" % (G, D, group_size))
    dq = torch.empty_like(q) if need_dq else None
    dk = torch.empty_like(q) if need_dkv else None
    dv = torch.empty_like(q) if need_dkv else None
    dh = torch.empty((G, l_h), dtype=torch.float32, device=dev) if need_dh else None
    ws = None
    ws_n = 0
    if need_dh:
        ws_n = bwd_workspace_bytes(B, L, D, group_size, l_h, code)
        ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: t.data_ptr() if t is not None else None
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), dy.data_ptr(), B, L, D,
            group_size, l_h, ptr(dq), ptr(dk), ptr(dv), ptr(dh), ptr(ws), ws_n, code,
            stream.cuda_stream)
    if dev.index == torch.cuda.current_device():
        st = lib().hyena_conv_bwd(*args)
    else:
        with torch.cuda.device(dev):
            st = lib().hyena_conv_bwd(*args)
    if st != 0:
        raise HyenaError(st, "hyena_conv_bwd")
    return dq, dk, dv, dh


def long_workspace_bytes(B: int, L: int, D: int, group_size: int, l_h: int,
                         dtype: int = DTYPE_BF16) -> int:
    """Workspace bytes hyena_conv_fwd_long needs (FFT work area and filter spectra)."""
    n = ctypes.c_int64()
    st = lib().hyena_conv_fwd_long_workspace(B, L, D, group_size, l_h, dtype, ctypes.byref(n))
    if st != 0:
        raise HyenaError(st, "hyena_conv_fwd_long_workspace")
    return n.value


def conv_fwd_long(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, h: torch.Tensor,
                  group_size: int, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None,
                  reuse_spectra: bool = False) -> torch.Tensor:
    """y = q (.) (h * (k (.) v)) by FFT convolution, for filters of any length.

    Same tensors as conv_fwd; h is [D // group_size, l_h] with any l_h >= 1.
    ``workspace`` (uint8, on q's device) is allocated here if not given.
    ``reuse_spectra``: the workspace already holds h's spectra from an
    earlier call with the same h, L and sizes (hyena_conv_fwd_long_ex).
    """
    dt, dev = q.dtype, q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("h", h)):
        if t.dtype != dt or t.device != dev or dev.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor like q" % name)
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or h.dim() != 2:
        raise ValueError("q, k, v must be [B, L, D]; h [D // group_size, l_h]")
    code = _dtype_code(dt)
    B, L, D = q.shape
    G, l_h = h.shape
    if group_size < 1 or D % group_size != 0 or G != D // group_size:
        raise ValueError("h has %d filters; D=%d, group_size=%d" % (G, D, group_size))
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != dt or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    ws_n = long_workspace_bytes(B, L, D, group_size, l_h, code)
    if reuse_spectra and workspace is None:
        raise ValueError("reuse_spectra needs the workspace of an earlier call")
    if workspace is None:
        workspace = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < ws_n:
        raise ValueError("workspace must hold %d bytes on q's device" % ws_n)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), B, L, D, group_size, l_h,
            out.data_ptr(), code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            int(bool(reuse_spectra)), stream.cuda_stream)
    if dev.index == torch.cuda.current_device():
        st = lib().hyena_conv_fwd_long_ex(*args)
    else:
        with torch.cuda.device(dev):
            st = lib().hyena_conv_fwd_long_ex(*args)
    if st != 0:
        raise HyenaError(st, "hyena_conv_fwd_long_ex")
    return out


def bwd_long_workspace_bytes(B: int, L: int, D: int, group_size: int, l_h: int,
                             dtype: int = DTYPE_BF16) -> int:
    """Workspace bytes hyena_conv_bwd_long needs."""
    n = ctypes.c_int64()
    st = lib().hyena_conv_bwd_long_workspace(B, L, D, group_size, l_h, dtype, ctypes.byref(n))
    if st != 0:
        raise HyenaError(st, "hyena_conv_bwd_long_workspace")
    return n.value


def conv_bwd_long(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, h: torch.Tensor,
                  dy: torch.Tensor, group_size: int, need_dq: bool = True, need_dkv: bool = True,
                  need_dh: bool = True, workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None, reuse_spectra: bool = False):
    """Gradients (dq, dk, dv, dh) of the long-filter forward (FFT), any l_h.

    Same tensors and results as conv_bwd; parts not requested are None.
    ``workspace`` (uint8, on q's device) is allocated here if not given.
    ``reuse_spectra``: the workspace already holds h's spectra from an
    earlier conv_fwd_long or conv_bwd_long call on it with the same h and
    sizes (hyena_conv_bwd_long_ex).
    """
    dt, dev = q.dtype, q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("h", h), ("dy", dy)):
        if t.dtype != dt or t.device != dev or dev.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor like q" % name)
    if q.dim() != 3 or any(t.shape != q.shape for t in (k, v, dy)) or h.dim() != 2:
        raise ValueError("q, k, v, dy must be [B, L, D]; h [D // group_size, l_h]")
    code = _dtype_code(dt)
    B, L, D = q.shape
    G, l_h = h.shape
    if group_size < 1 or D % group_size != 0 or G != D // group_size:
        raise ValueError("h has %d filters; D=%d, group_size=%d" % (G, D, group_size))
    dq = torch.empty_like(q) if need_dq else None
    dk = torch.empty_like(q) if need_dkv else None
    dv = torch.empty_like(q) if need_dkv else None
    dh = torch.empty((G, l_h), dtype=torch.float32, device=dev) if need_dh else None
    ws_n = bwd_long_workspace_bytes(B, L, D, group_size, l_h, code)
    if reuse_spectra and workspace is None:
        raise ValueError("reuse_spectra needs the workspace of an earlier call")
    if workspace is None:
        workspace = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < ws_n:
        raise ValueError("workspace must hold %d bytes on q's device" % ws_n)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: t.data_ptr() if t is not None else None
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), dy.data_ptr(), B, L, D,
            group_size, l_h, ptr(dq), ptr(dk), ptr(dv), ptr(dh), code, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), int(bool(reuse_spectra)), stream.cuda_stream)
    if dev.index == torch.cuda.current_device():
        st = lib().hyena_conv_bwd_long_ex(*args)
    else:
        with torch.cuda.device(dev):
            st = lib().hyena_conv_bwd_long_ex(*args)
    if st != 0:
        raise HyenaError(st, "hyena_conv_bwd_long_ex")
    return dq, dk, dv, dh


MAX_DIRECT_TAPS = 2 * BLOCK_LEN  # longest filter of the chunked kernels (128)


class HyenaConv(torch.autograd.Function):
    """Autograd wrapper: y = HyenaConv.apply(q, k, v, h, group_size).

    Filters of up to MAX_DIRECT_TAPS taps run on the chunked kernels; longer
    ones on the FFT path (as HyenaConvLong).  The filter gradient comes back
    in h's dtype (accumulated in fp32).
    """

    @staticmethod
    def forward(ctx, q, k, v, h, group_size):
        if h.dim() == 2 and h.shape[1] > MAX_DIRECT_TAPS:
            ctx.long = True
            return HyenaConvLong.forward(ctx, q, k, v, h, group_size)
        ctx.long = False
        ctx.save_for_backward(q, k, v, h)
        ctx.group_size = group_size
        return conv_fwd(q, k, v, h, group_size)

    @staticmethod
    def backward(ctx, dy):
        if ctx.long:
            return HyenaConvLong.backward(ctx, dy)
        q, k, v, h = ctx.saved_tensors
        need = ctx.needs_input_grad
        dq, dk, dv, dh = conv_bwd(q, k, v, h, dy.contiguous(), ctx.group_size,
                                  need_dq=need[0], need_dkv=need[1] or need[2], need_dh=need[3])
        return (dq, dk if need[1] else None, dv if need[2] else None,
                dh.to(h.dtype) if dh is not None else None, None)


class HyenaConvLong(torch.autograd.Function):
    """Autograd wrapper of the long-filter (FFT) path: y = HyenaConvLong.apply(q, k, v, h, group_size).

    Any filter length; the filter gradient comes back in h's dtype (fp32 sums).
    The forward runs in a workspace of the backward's size, kept until the
    backward, which then reuses the filter spectra the forward left in it.
    """

    @staticmethod
    def forward(ctx, q, k, v, h, group_size):
        ctx.save_for_backward(q, k, v, h)
        ctx.group_size = group_size
        B, L, D = q.shape
        n = bwd_long_workspace_bytes(B, L, D, group_size, h.shape[1], _dtype_code(q.dtype))
        ctx.workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
        return conv_fwd_long(q, k, v, h, group_size, workspace=ctx.workspace)

    @staticmethod
    def backward(ctx, dy):
        q, k, v, h = ctx.saved_tensors
        need = ctx.needs_input_grad
        dq, dk, dv, dh = conv_bwd_long(q, k, v, h, dy.contiguous(), ctx.group_size,
                                       need_dq=need[0], need_dkv=need[1] or need[2],
                                       need_dh=need[3], workspace=ctx.workspace,
                                       reuse_spectra=True)
        ctx.workspace = None
        return (dq, dk if need[1] else None, dv if need[2] else None,
                dh.to(h.dtype) if dh is not None else None, None)
