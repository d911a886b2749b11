"""Thin ctypes binding of libpsa_attn.so.

The names mirror the C ABI in include/psa_attn.h one to one and only marshal
arguments; every step of the computation runs in the HIP kernels.  PyTorch is
used for device memory and the current stream, nothing else.  There is no
fallback: if the library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

PSA_F32 = 0
PSA_BF16 = 1
PSA_F16 = 2

STATUS = {0: "PSA_OK", 1: "PSA_ERR_NULL", 2: "PSA_ERR_SHAPE", 3: "PSA_ERR_UNSUPPORTED",
          4: "PSA_ERR_ALIGN", 5: "PSA_ERR_ALIAS", 6: "PSA_ERR_NOMEM", 7: "PSA_ERR_HIP",
          8: "PSA_ERR_DEVICE"}

EXPORTS = ("psa_attn_fwd", "psa_attn_bwd", "psa_attn_bwd_noalloc", "psa_attn_fwd_vslice", "psa_attn_bwd_vslice", "psa_merge_fwd",
           "psa_merge_bwd", "psa_qkv_conv_bwd", "psa_qkv_conv_cat_bwd",
           "psa_channel_cat_bwd", "psa_attn_supported", "psa_last_error",
           "psa_attn_version", "psa_attn_timing_enable", "psa_attn_timing_read",
           "psa_attn_timing_reset")
TIMING_SLOTS = ("fwd", "bwd_pre", "bwd_main", "reserved", "conv_dx", "conv_dw", "cat", "merge_fwd", "merge_bwd")

_lib = None


class PsaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS.get(code, code)}: {msg}")
        self.code = code


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the library; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("PSA_ATTN_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with vision_transformer_attention_psa_amd.build "
                           "(or __graft_entry__.build()) before use")
    lib = ctypes.CDLL(p)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.psa_attn_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.psa_attn_fwd.restype = i
    lib.psa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.psa_attn_bwd.restype = i
    lib.psa_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.psa_attn_bwd_noalloc.restype = i
    lib.psa_attn_fwd_vslice.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.psa_attn_fwd_vslice.restype = i
    lib.psa_attn_bwd_vslice.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    lib.psa_attn_bwd_vslice.restype = i
    lib.psa_merge_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    lib.psa_merge_fwd.restype = i
    lib.psa_merge_bwd.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    lib.psa_merge_bwd.restype = i
    lib.psa_qkv_conv_bwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.psa_qkv_conv_bwd.restype = i
    lib.psa_qkv_conv_cat_bwd.argtypes = [vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(i), i, vp, i, i, i,
                                         i, i, vp]
    lib.psa_qkv_conv_cat_bwd.restype = i
    lib.psa_channel_cat_bwd.argtypes = [vp, vp, i, i, i, i, i, vp]
    lib.psa_channel_cat_bwd.restype = i
    lib.psa_attn_supported.argtypes = [i, i, i]
    lib.psa_attn_supported.restype = i
    lib.psa_last_error.argtypes = []
    lib.psa_last_error.restype = ctypes.c_char_p
    lib.psa_attn_version.argtypes = []
    lib.psa_attn_version.restype = i
    lib.psa_attn_timing_enable.argtypes = [i]
    lib.psa_attn_timing_enable.restype = i
    lib.psa_attn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_longlong), i]
    lib.psa_attn_timing_read.restype = i
    lib.psa_attn_timing_reset.argtypes = []
    lib.psa_attn_timing_reset.restype = i
    if path is None:
        _lib = lib
    return lib


def psa_last_error() -> str:
    return load().psa_last_error().decode()


def psa_attn_supported(dk: int, dv: int, dtype: int) -> bool:
    return bool(load().psa_attn_supported(dk, dv, dtype))


def psa_attn_version() -> int:
    return load().psa_attn_version()


def psa_attn_timing_enable(on: bool) -> int:
    return load().psa_attn_timing_enable(1 if on else 0)


def psa_attn_timing_reset() -> int:
    return load().psa_attn_timing_reset()


def psa_attn_timing_read() -> dict:
    """{slot: (total_ms, launches)} for every kernel slot."""
    n = len(TIMING_SLOTS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_longlong * n)()
    _check("psa_attn_timing_read", load().psa_attn_timing_read(ms, cnt, n))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(TIMING_SLOTS)}


def psa_attn_fwd(qkv: int, o: int, lse: int, B: int, heads: int, N: int, dk: int, dv: int,
                 scale: float, dtype: int, stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_attn_fwd(qkv, o, lse, B, heads, N, dk, dv, scale, dtype, stream)


def psa_attn_bwd(qkv: int, o: int, lse: int, dO: int, d_packed: int, B: int, heads: int, N: int,
                 dk: int, dv: int, scale: float, dtype: int, stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_attn_bwd(qkv, o, lse, dO, d_packed, B, heads, N, dk, dv, scale, dtype, stream)


def psa_attn_bwd_noalloc(qkv: int, o: int, lse: int, dO: int, d_packed: int, B: int, heads: int, N: int,
                         dk: int, dv: int, scale: float, dtype: int, stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_attn_bwd_noalloc(qkv, o, lse, dO, d_packed, B, heads, N, dk, dv, scale, dtype, stream)


def psa_attn_fwd_vslice(qkv: int, o: int, lse: int, B: int, heads: int, N: int, dk: int, dv_total: int, v0: int,
                        dv: int, scale: float, dtype: int, stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_attn_fwd_vslice(qkv, o, lse, B, heads, N, dk, dv_total, v0, dv, scale, dtype, stream)


def psa_attn_bwd_vslice(qkv: int, o: int, lse: int, dO: int, d_packed: int, B: int, heads: int, N: int, dk: int,
                        dv_total: int, v0: int, dv: int, accumulate: int, scale: float, dtype: int,
                        stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_attn_bwd_vslice(qkv, o, lse, dO, d_packed, B, heads, N, dk, dv_total, v0, dv, accumulate,
                                      scale, dtype, stream)


def psa_merge_fwd(o_lo: int, o_hi: int, merged: int, B: int, heads: int, N: int, half: int, dtype: int,
                  stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_merge_fwd(o_lo, o_hi, merged, B, heads, N, half, dtype, stream)


def psa_merge_bwd(d_merged: int, d_lo: int, d_hi: int, B: int, heads: int, N: int, half: int, dtype: int,
                  stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_merge_bwd(d_merged, d_lo, d_hi, B, heads, N, half, dtype, stream)


# ------------------------------------------------------------ torch helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PSA_F32
    if t.dtype == torch.bfloat16:
        return PSA_BF16
    if t.dtype == torch.float16:
        return PSA_F16
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise PsaError(fn, rc, psa_last_error())


def _stream(t) -> int:
    """Handle of torch's current stream on t's device.  torch's raw accessor
    returns it without building a Stream object (about 2 us per call less);
    the public call is the fallback."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.device.index if t.device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _on_gpu(fn: str, *named) -> None:
    """Every tensor must live on one GPU.  The library receives raw addresses,
    and a host address handed to a kernel is a GPU memory fault, so this is
    checked before any library call (and again by the library itself)."""
    dev = None
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{fn}: {name} is on {t.device}; every tensor must be on a GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{fn}: {name} is on {t.device} but {named[0][0]} is on {dev}; "
                             "every tensor must be on one GPU")


def _check_out(name: str, t, shape, dtype, device) -> None:
    """Caller-provided outputs must be exactly what the library will write."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"out {name} must be a contiguous {tuple(shape)} {dtype} tensor on {device}; "
                         f"got {tuple(t.shape)} {t.dtype} on {t.device}")


def psa_qkv_conv_bwd(x: int, w: int, dy: int, dx: int, dw: int, B: int, cin: int, cout: int, N: int,
                     dtype: int, stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_qkv_conv_bwd(x, w, dy, dx, dw, B, cin, cout, N, dtype, stream)


def psa_qkv_conv_cat_bwd(x: int, w: int, dy: int, dx_parts, part_channels, dw: int, B: int, cin: int,
                         cout: int, N: int, dtype: int, stream: int | None) -> int:
    """Raw call; dx_parts (device addresses) and part_channels are Python
    sequences of equal length.  Returns the status code."""
    n = len(dx_parts)
    ptrs = (ctypes.c_void_p * max(1, n))(*dx_parts)
    chans = (ctypes.c_int * max(1, len(part_channels)))(*part_channels)
    return load().psa_qkv_conv_cat_bwd(x, w, dy, ptrs, chans, n, dw, B, cin, cout, N, dtype, stream)


def psa_channel_cat_bwd(dy: int, dx: int, n_outer: int, chunk: int, total: int, offset: int, dtype: int,
                        stream: int | None) -> int:
    """Raw call with device addresses; returns the status code."""
    return load().psa_channel_cat_bwd(dy, dx, n_outer, chunk, total, offset, dtype, stream)


def _shape(qkv, dk: int, dv: int):
    if qkv.dim() != 4 or qkv.shape[2] != 2 * dk + dv:
        raise ValueError(f"qkv must be [B, heads, 2*dk+dv, N]; got {tuple(qkv.shape)}")
    if not qkv.is_contiguous():
        raise ValueError("qkv must be contiguous")
    B, H, _, N = qkv.shape
    return B, H, N


def fwd(qkv, dk: int, dv: int, scale: float, out=None):
    """O [B, heads, dv, N] (qkv's dtype) and LSE [B, heads, N] (float32)."""
    import torch
    B, H, N = _shape(qkv, dk, dv)
    _on_gpu("fwd", ("qkv", qkv))
    if out is None:
        o = torch.empty((B, H, dv, N), dtype=qkv.dtype, device=qkv.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=qkv.device)
    else:
        o, lse = out
        _on_gpu("fwd", ("qkv", qkv), ("o", o), ("lse", lse))
        _check_out("o", o, (B, H, dv, N), qkv.dtype, qkv.device)
        _check_out("lse", lse, (B, H, N), torch.float32, qkv.device)
    _check("psa_attn_fwd", psa_attn_fwd(qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, dk,
                                        dv, float(scale), _dtype_code(qkv), _stream(qkv)))
    return o, lse


def bwd(qkv, o, lse, dO, dk: int, dv: int, scale: float, out=None):
    """d_packed [B, heads, 2dk+dv, N]: sections dQ, dK, dV."""
    import torch
    B, H, N = _shape(qkv, dk, dv)
    _on_gpu("bwd", ("qkv", qkv), ("o", o), ("lse", lse), ("dO", dO), *((("out", out),) if out is not None else ()))
    for name, t in (("o", o), ("lse", lse), ("dO", dO)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tuple(o.shape) != (B, H, dv, N) or tuple(dO.shape) != (B, H, dv, N):
        raise ValueError("o and dO must be [B, heads, dv, N]")
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, heads, N]")
    if o.dtype != qkv.dtype or dO.dtype != qkv.dtype:
        raise ValueError("o and dO must have qkv's dtype")
    d = torch.empty_like(qkv) if out is None else out
    _check_out("d_packed", d, qkv.shape, qkv.dtype, qkv.device)
    _check("psa_attn_bwd", psa_attn_bwd(qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), dO.data_ptr(),
                                        d.data_ptr(), B, H, N, dk, dv, float(scale),
                                        _dtype_code(qkv), _stream(qkv)))
    return d


def conv_bwd(x, w, dy, out=None):
    """(dx [B, cin, N], dw [cout, cin]) of the 1x1 convolution y = w x, for
    x [B, cin, N], w [cout, cin] and dy [B, cout, N] (dy may be a packed
    gradient [B, heads, 2dk+dv, N]; it is read as [B, cout, N])."""
    import torch
    if x.dim() != 3 or w.dim() != 2:
        raise ValueError("x must be [B, cin, N] and w [cout, cin]")
    B, cin, N = x.shape
    cout = w.shape[0]
    if w.shape[1] != cin or dy.numel() != B * cout * N or dy.shape[0] != B or dy.shape[-1] != N:
        raise ValueError(f"dy must hold [B, cout, N] = [{B}, {cout}, {N}]; got {tuple(dy.shape)}")
    _on_gpu("conv_bwd", ("x", x), ("w", w), ("dy", dy))
    for name, t in (("x", x), ("w", w), ("dy", dy)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != x.dtype:
            raise ValueError("x, w and dy must share one dtype")
    if out is None:
        dx = torch.empty_like(x)
        dw = torch.empty_like(w)
    else:
        dx, dw = out
        _on_gpu("conv_bwd", ("x", x), ("dx", dx), ("dw", dw))
        _check_out("dx", dx, x.shape, x.dtype, x.device)
        _check_out("dw", dw, w.shape, w.dtype, x.device)
    _check("psa_qkv_conv_bwd", psa_qkv_conv_bwd(x.data_ptr(), w.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                                                dw.data_ptr(), B, cin, cout, N, _dtype_code(x), _stream(x)))
    return dx, dw


def conv_cat_bwd(x, w, dy, part_channels, out=None):
    """([dx_k [B, c_k, N] for each part], dw [cout, cin]) of y = w cat(x_0, ...)
    for the concatenated input x [B, cin, N]; sum(part_channels) == cin."""
    import torch
    if x.dim() != 3 or w.dim() != 2:
        raise ValueError("x must be [B, cin, N] and w [cout, cin]")
    B, cin, N = x.shape
    cout = w.shape[0]
    if w.shape[1] != cin or dy.numel() != B * cout * N or dy.shape[0] != B or dy.shape[-1] != N:
        raise ValueError(f"dy must hold [B, cout, N] = [{B}, {cout}, {N}]; got {tuple(dy.shape)}")
    _on_gpu("conv_cat_bwd", ("x", x), ("w", w), ("dy", dy))
    for name, t in (("x", x), ("w", w), ("dy", dy)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != x.dtype:
            raise ValueError("x, w and dy must share one dtype")
    if out is None:
        dxs = [torch.empty((B, c, N), dtype=x.dtype, device=x.device) for c in part_channels]
        dw = torch.empty_like(w)
    else:
        dxs, dw = out
        if len(dxs) != len(part_channels):
            raise ValueError("out must hold one dx tensor per part")
        _on_gpu("conv_cat_bwd", ("x", x), ("dw", dw), *((f"dx[{k}]", d_) for k, d_ in enumerate(dxs)))
        for k, (d_, c) in enumerate(zip(dxs, part_channels)):
            _check_out(f"dx[{k}]", d_, (B, c, N), x.dtype, x.device)
        _check_out("dw", dw, w.shape, w.dtype, x.device)
    _check("psa_qkv_conv_cat_bwd",
           psa_qkv_conv_cat_bwd(x.data_ptr(), w.data_ptr(), dy.data_ptr(), [d.data_ptr() for d in dxs],
                                list(part_channels), dw.data_ptr(), B, cin, cout, N, _dtype_code(x),
                                _stream(x)))
    return dxs, dw


def channel_cat_bwd(dy, channels: int, offset: int, out=None):
    """dx [B, channels, *spatial] = dy[:, offset:offset + channels] for a
    contiguous channel-concatenated gradient dy [B, C, *spatial]."""
    import torch
    if dy.dim() < 2 or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous [B, C, ...] tensor")
    _on_gpu("channel_cat_bwd", ("dy", dy), *((("out", out),) if out is not None else ()))
    B, C = dy.shape[0], dy.shape[1]
    inner = dy[0, 0].numel()
    shape = (B, channels, *dy.shape[2:])
    dx = torch.empty(shape, dtype=dy.dtype, device=dy.device) if out is None else out
    if tuple(dx.shape) != shape or dx.dtype != dy.dtype or not dx.is_contiguous():
        raise ValueError(f"out must be a contiguous {shape} tensor of dy's dtype")
    _check("psa_channel_cat_bwd", psa_channel_cat_bwd(dy.data_ptr(), dx.data_ptr(), B, channels * inner,
                                                      C * inner, offset * inner, _dtype_code(dy),
                                                      _stream(dy)))
    return dx


def _vslice_shape(qkv, dk: int, dv_total: int):
    if qkv.dim() != 4 or qkv.shape[2] != 2 * dk + dv_total:
        raise ValueError(f"qkv must be [B, heads, 2*dk+dv_total, N]; got {tuple(qkv.shape)}")
    if not qkv.is_contiguous():
        raise ValueError("qkv must be contiguous")
    B, H, _, N = qkv.shape
    return B, H, N


def fwd_vslice(qkv, dk: int, dv_total: int, v0: int, dv: int, scale: float, out=None):
    """Attention over V rows [v0, v0+dv): O [B, heads, dv, N] and LSE [B, heads, N]."""
    import torch
    B, H, N = _vslice_shape(qkv, dk, dv_total)
    _on_gpu("fwd_vslice", ("qkv", qkv))
    if out is None:
        o = torch.empty((B, H, dv, N), dtype=qkv.dtype, device=qkv.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=qkv.device)
    else:
        o, lse = out
        _on_gpu("fwd_vslice", ("qkv", qkv), ("o", o), ("lse", lse))
        _check_out("o", o, (B, H, dv, N), qkv.dtype, qkv.device)
        _check_out("lse", lse, (B, H, N), torch.float32, qkv.device)
    _check("psa_attn_fwd_vslice", psa_attn_fwd_vslice(qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, dk,
                                                      dv_total, v0, dv, float(scale), _dtype_code(qkv),
                                                      _stream(qkv)))
    return o, lse


def bwd_vslice(qkv, o, lse, dO, d_packed, dk: int, dv_total: int, v0: int, dv: int, scale: float,
               accumulate: bool):
    """Backward of one V-slice call into d_packed (in place): dV rows of the
    slice overwritten, dQ and dK overwritten or (accumulate) added to."""
    import torch
    B, H, N = _vslice_shape(qkv, dk, dv_total)
    _on_gpu("bwd_vslice", ("qkv", qkv), ("o", o), ("lse", lse), ("dO", dO), ("d_packed", d_packed))
    for name, t in (("o", o), ("lse", lse), ("dO", dO), ("d_packed", d_packed)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tuple(o.shape) != (B, H, dv, N) or tuple(dO.shape) != (B, H, dv, N):
        raise ValueError("o and dO must be [B, heads, dv, N]")
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, heads, N]")
    if tuple(d_packed.shape) != tuple(qkv.shape):
        raise ValueError("d_packed must have qkv's shape")
    for t in (o, dO, d_packed):
        if t.dtype != qkv.dtype:
            raise ValueError("o, dO and d_packed must have qkv's dtype")
    _check("psa_attn_bwd_vslice",
           psa_attn_bwd_vslice(qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), dO.data_ptr(), d_packed.data_ptr(),
                               B, H, N, dk, dv_total, v0, dv, 1 if accumulate else 0, float(scale),
                               _dtype_code(qkv), _stream(qkv)))
    return d_packed


def merge_fwd(o_lo, o_hi, out=None):
    """merged [B, heads, 2*half, N]: each head's lo channels, then its hi ones."""
    import torch
    if o_lo.dim() != 4 or o_lo.shape != o_hi.shape or o_lo.dtype != o_hi.dtype:
        raise ValueError("o_lo and o_hi must be equal-shaped [B, heads, half, N]")
    if not (o_lo.is_contiguous() and o_hi.is_contiguous()):
        raise ValueError("o_lo and o_hi must be contiguous")
    _on_gpu("merge_fwd", ("o_lo", o_lo), ("o_hi", o_hi), *((("out", out),) if out is not None else ()))
    B, H, half, N = o_lo.shape
    m = torch.empty((B, H, 2 * half, N), dtype=o_lo.dtype, device=o_lo.device) if out is None else out
    _check_out("merged", m, (B, H, 2 * half, N), o_lo.dtype, o_lo.device)
    _check("psa_merge_fwd", psa_merge_fwd(o_lo.data_ptr(), o_hi.data_ptr(), m.data_ptr(), B, H, N, half,
                                          _dtype_code(o_lo), _stream(o_lo)))
    return m


def merge_bwd(d_merged, out=None):
    """(d_lo, d_hi) [B, heads, half, N] from d_merged [B, heads, 2*half, N]."""
    import torch
    if d_merged.dim() != 4 or d_merged.shape[2] % 2 or not d_merged.is_contiguous():
        raise ValueError("d_merged must be a contiguous [B, heads, 2*half, N] tensor")
    _on_gpu("merge_bwd", ("d_merged", d_merged), *((("d_lo", out[0]), ("d_hi", out[1])) if out is not None else ()))
    B, H, C, N = d_merged.shape
    half = C // 2
    if out is None:
        lo = torch.empty((B, H, half, N), dtype=d_merged.dtype, device=d_merged.device)
        hi = torch.empty_like(lo)
    else:
        lo, hi = out
        _check_out("d_lo", lo, (B, H, half, N), d_merged.dtype, d_merged.device)
        _check_out("d_hi", hi, (B, H, half, N), d_merged.dtype, d_merged.device)
    _check("psa_merge_bwd", psa_merge_bwd(d_merged.data_ptr(), lo.data_ptr(), hi.data_ptr(), B, H, N, half,
                                          _dtype_code(d_merged), _stream(d_merged)))
    return lo, hi


def _autograd_function():
    import torch

    class PsaAttnFunction(torch.autograd.Function):
        """O = PSA attention of the packed qkv [B, heads, 2dk+dv, N]; the
        backward returns d_packed through psa_attn_bwd (deterministic)."""

        @staticmethod
        def forward(ctx, qkv, dk: int, dv: int, scale: float):
            qkv = qkv.contiguous()
            o, lse = fwd(qkv, dk, dv, scale)
            ctx.save_for_backward(qkv, o, lse)
            ctx.dims = (dk, dv, scale)
            return o

        @staticmethod
        def backward(ctx, dO):
            qkv, o, lse = ctx.saved_tensors
            dk, dv, scale = ctx.dims
            return bwd(qkv, o, lse, dO.contiguous(), dk, dv, scale), None, None, None

    return PsaAttnFunction


_FN = None


def psa_attention(qkv, dk: int, dv: int, scale: float):
    """Differentiable PSA attention: O [B, heads, dv, N] from qkv."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    return _FN.apply(qkv, dk, dv, scale)
