"""Thin ctypes binding of libmoe.so (declared in include/moe.h).

Functions keep the C names and only marshal arguments: torch tensors become
device pointers, the current torch stream becomes the hipStream_t, and a
non-OK status becomes :class:`MoEError`. Every step of the layer runs in the
library's HIP kernels; if the library is missing this module raises, it never
falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

PRECISIONS = {"bf16": 0, "fp8_block": 1, "mxfp8": 2, "fp8_bwd": 3, "fp8_fp4": 4, "fp8_block_f32": 5,
              "fp8_bwd_f32": 6}

STATUS_NAMES = {
    0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
    4: "MOE_ERR_PRECISION", 5: "MOE_ERR_ARCH", 6: "MOE_ERR_WORKSPACE",
    7: "MOE_ERR_LAUNCH", 8: "MOE_ERR_ROUTING", 9: "MOE_ERR_UNSUPPORTED",
}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {moe_status_string(status)}")


MOE_FLAG_FP8_WGRAD = 1
WGRADS = {"bf16": 0, "fp8": MOE_FLAG_FP8_WGRAD}


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64),
                ("precision", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class moe_saved_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("counts", "offsets", "row_of", "src_of", "wrow", "h13", "act", "total")]


class moe_wq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("w13", "w13_scale", "w2", "w2_scale", "w2t", "w2t_scale", "w13t", "w13t_scale", "total")]


class moe_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "moe_workspace_size": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_get_saved_layout": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.POINTER(moe_saved_layout)]),
    "moe_get_wq_layout": (ctypes.c_int, [ctypes.POINTER(moe_shape), ctypes.POINTER(moe_wq_layout)]),
    "moe_quantize_weights": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P]),
    "moe_quantize_rows": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                         _P]),
    "moe_quantize_tokens": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, ctypes.c_int64, ctypes.c_int64, _P,
                                           _P, _P, _P, _P, _P]),
    "moe_permute_scratch_bytes": (ctypes.c_size_t, [ctypes.POINTER(moe_shape)]),
    "moe_permute": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P]),
    "moe_fwd": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               ctypes.c_size_t, _P]),
    "moe_fwd_logits": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                      _P, _P, ctypes.c_size_t, _P]),
    "moe_bwd": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _P, ctypes.c_size_t, _P]),
    "moe_permute_noalloc": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, _P, _P, _P]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, ctypes.c_int32, _P, _P, _P]),
    "moe_route_bwd": (ctypes.c_int, [ctypes.POINTER(moe_shape), _P, _P, _P, _P, ctypes.c_int32, _P, _P]),
    "moe_read_status": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int32), _P]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_set_kernel_timing": (ctypes.c_int, [ctypes.c_int]),
    "moe_kernel_timing_collect": (ctypes.c_int, [ctypes.POINTER(moe_kernel_time), ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_int32)]),
}


def lib() -> ctypes.CDLL:
    """Loads libmoe.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m grouped_gemm_02_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_symbols() -> list[str]:
    return list(_SIGS)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoEError(status, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


MOE_ERR_SHAPE = 2


def _want(t, name: str, dtype, numel: int | None = None, optional: bool = False) -> None:
    """Checks a tensor argument before its pointer crosses the C ABI, which
    cannot see dtypes, strides or sizes: it must be a contiguous GPU tensor of
    `dtype` with at least `numel` elements. Raises MoEError(MOE_ERR_SHAPE)
    otherwise. Anything that is not a torch tensor (None, a raw address) is
    passed through for the library's own checks (NULL, alignment)."""
    if not isinstance(t, torch.Tensor):
        return
    if t.dtype != dtype:
        raise MoEError(MOE_ERR_SHAPE, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise MoEError(MOE_ERR_SHAPE, f"{name} is not contiguous")
    if numel is not None and t.numel() < numel:
        raise MoEError(MOE_ERR_SHAPE, f"{name} holds {t.numel()} elements, needs {numel}")
    if t.device.type != "cuda":
        raise MoEError(MOE_ERR_SHAPE, f"{name} is on {t.device}, expected a GPU tensor")


_BF16, _I32, _F32, _U8 = torch.bfloat16, torch.int32, torch.float32, torch.uint8


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_shape(T, H, I, E, k, precision="bf16", num_cus=0, wgrad="bf16") -> moe_shape:
    """wgrad: "bf16" (default) or "fp8" (sets MOE_FLAG_FP8_WGRAD)."""
    p = PRECISIONS[precision] if isinstance(precision, str) else int(precision)
    f = WGRADS[wgrad] if isinstance(wgrad, str) else int(wgrad)
    return moe_shape(int(T), int(H), int(I), int(E), int(k), p, int(num_cus), f, 0)


# ------------------------------------------------------------ C entry points

def moe_status_string(status: int) -> str:
    try:
        return lib().moe_status_string(int(status)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(int(status), f"status {status}")


def moe_workspace_size(shape: moe_shape):
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(shape), ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)),
           "moe_workspace_size")
    return f.value, s.value, b.value


def moe_get_saved_layout(shape: moe_shape) -> dict:
    out = moe_saved_layout()
    _check(lib().moe_get_saved_layout(ctypes.byref(shape), ctypes.byref(out)), "moe_get_saved_layout")
    return {n: getattr(out, n) for n, _ in moe_saved_layout._fields_}


def moe_get_wq_layout(shape: moe_shape) -> dict:
    out = moe_wq_layout()
    _check(lib().moe_get_wq_layout(ctypes.byref(shape), ctypes.byref(out)), "moe_get_wq_layout")
    return {n: getattr(out, n) for n, _ in moe_wq_layout._fields_}


def moe_quantize_weights(shape, W13, W2, wq, stream=None) -> None:
    if shape.precision != PRECISIONS["bf16"]:
        E, H, I = shape.E, shape.H, shape.I
        _want(W13, "W13", _BF16, E * 2 * I * H)
        _want(W2, "W2", _BF16, E * H * I)
        _want(wq, "wq", _U8, moe_get_wq_layout(shape)["total"])
    _check(lib().moe_quantize_weights(ctypes.byref(shape), _ptr(W13), _ptr(W2), _ptr(wq), _stream(stream)),
           "moe_quantize_weights")


def wgrad_rows_cap(shape: moe_shape) -> int:
    """K of moe_quantize_tokens' buffers: codes C*K bytes, scales C*K/32."""
    return 128 * (shape.T * shape.k // 128 + shape.E)


def moe_quantize_tokens(shape, x, ld, C, counts, offsets, src_of, codes, scales, stream=None) -> None:
    if shape.T > 0:
        K = wgrad_rows_cap(shape)
        _want(x, "in", _BF16)
        _want(counts, "counts", _I32, shape.E)
        _want(offsets, "offsets", _I32, shape.E + 1)
        _want(src_of, "src_of", _I32, shape.T * shape.k, optional=True)
        _want(codes, "codes", _U8, int(C) * K)
        _want(scales, "scales", _U8, int(C) * K // 32)
    _check(lib().moe_quantize_tokens(ctypes.byref(shape), _ptr(x), int(ld), int(C), _ptr(counts), _ptr(offsets),
                                     _ptr(src_of), _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_tokens")


def moe_quantize_rows(shape, x, rows, K, codes, scales, stream=None) -> None:
    if rows > 0:
        _want(x, "in", _BF16, int(rows) * int(K))
        _want(codes, "codes", _U8, int(rows) * int(K))
        _want(scales, "scales", _U8, int(rows) * int(K) // 32)
    _check(lib().moe_quantize_rows(ctypes.byref(shape), _ptr(x), int(rows), int(K), _ptr(codes), _ptr(scales),
                                   _stream(stream)), "moe_quantize_rows")


def moe_permute_scratch_bytes(shape: moe_shape) -> int:
    return int(lib().moe_permute_scratch_bytes(ctypes.byref(shape)))


def moe_permute(shape, topk_idx, counts, offsets, row_of, src_of, scratch, stream=None) -> None:
    Tk = shape.T * shape.k
    _want(topk_idx, "topk_idx", _I32, Tk, optional=Tk == 0)
    _want(counts, "counts", _I32, shape.E)
    _want(offsets, "offsets", _I32, shape.E + 1)
    _want(row_of, "row_of", _I32, Tk, optional=Tk == 0)
    _want(src_of, "src_of", _I32, Tk, optional=Tk == 0)
    _want(scratch, "scratch", _U8, moe_permute_scratch_bytes(shape))
    _check(lib().moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(row_of),
                             _ptr(src_of), _ptr(scratch), _stream(stream)), "moe_permute")


def moe_permute_noalloc(shape, topk_idx, counts, offsets, row_of, src_of, status, stream=None) -> None:
    Tk = shape.T * shape.k
    _want(topk_idx, "topk_idx", _I32, Tk, optional=Tk == 0)
    _want(counts, "counts", _I32, shape.E)
    _want(offsets, "offsets", _I32, shape.E + 1)
    _want(row_of, "row_of", _I32, Tk, optional=Tk == 0)
    _want(src_of, "src_of", _I32, Tk, optional=Tk == 0)
    _want(status, "status", _I32, 1)
    _check(lib().moe_permute_noalloc(ctypes.byref(shape), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(row_of),
                                     _ptr(src_of), _ptr(status), _stream(stream)), "moe_permute_noalloc")


def moe_fwd(shape, x, topk_idx, topk_w, W13, W2, wq, y, saved, ws, stream=None) -> None:
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    f, s, _ = moe_workspace_size(shape)
    _want(x, "x", _BF16, T * H, optional=T == 0)
    _want(topk_idx, "topk_idx", _I32, T * k, optional=T == 0)
    _want(topk_w, "topk_w", _F32, T * k, optional=T == 0)
    _want(W13, "W13", _BF16, E * 2 * I * H)
    _want(W2, "W2", _BF16, E * H * I)
    _want(wq, "wq", _U8, moe_get_wq_layout(shape)["total"], optional=True)
    _want(y, "y", _BF16, T * H, optional=T == 0)
    _want(saved, "saved", _U8, s, optional=True)
    _want(ws, "ws", _U8, f)
    _check(lib().moe_fwd(ctypes.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W13), _ptr(W2),
                         _ptr(wq), _ptr(y), _ptr(saved), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)), "moe_fwd")


def moe_fwd_logits(shape, x, logits, renorm, topk_idx, topk_w, W13, W2, wq, y, saved, ws, stream=None) -> None:
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    f, s, _ = moe_workspace_size(shape)
    _want(x, "x", _BF16, T * H, optional=T == 0)
    _want(logits, "logits", _F32, T * E, optional=T == 0)
    _want(topk_idx, "topk_idx", _I32, T * k, optional=T == 0)
    _want(topk_w, "topk_w", _F32, T * k, optional=T == 0)
    _want(W13, "W13", _BF16, E * 2 * I * H)
    _want(W2, "W2", _BF16, E * H * I)
    _want(wq, "wq", _U8, moe_get_wq_layout(shape)["total"], optional=True)
    _want(y, "y", _BF16, T * H, optional=T == 0)
    _want(saved, "saved", _U8, s, optional=True)
    _want(ws, "ws", _U8, f)
    _check(lib().moe_fwd_logits(ctypes.byref(shape), _ptr(x), _ptr(logits), int(bool(renorm)), _ptr(topk_idx),
                                _ptr(topk_w), _ptr(W13), _ptr(W2), _ptr(wq), _ptr(y), _ptr(saved), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_fwd_logits")


def moe_bwd(shape, dy, x, topk_idx, topk_w, W13, W2, wq, saved, dx, d_topk_w, dW13, dW2, ws,
            stream=None) -> None:
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    _, s, b = moe_workspace_size(shape)
    for t, n, dt, cnt in ((dy, "dy", _BF16, T * H), (x, "x", _BF16, T * H), (topk_idx, "topk_idx", _I32, T * k),
                          (topk_w, "topk_w", _F32, T * k), (dx, "dx", _BF16, T * H),
                          (d_topk_w, "d_topk_w", _F32, T * k)):
        _want(t, n, dt, cnt, optional=T == 0)
    _want(W13, "W13", _BF16, E * 2 * I * H)
    _want(W2, "W2", _BF16, E * H * I)
    _want(wq, "wq", _U8, moe_get_wq_layout(shape)["total"], optional=True)
    _want(saved, "saved", _U8, s)
    _want(dW13, "dW13", _BF16, E * 2 * I * H)
    _want(dW2, "dW2", _BF16, E * H * I)
    _want(ws, "ws", _U8, b)
    _check(lib().moe_bwd(ctypes.byref(shape), _ptr(dy), _ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W13),
                         _ptr(W2), _ptr(wq), _ptr(saved), _ptr(dx), _ptr(d_topk_w), _ptr(dW13), _ptr(dW2),
                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_bwd")


def moe_route(shape, logits, renorm, topk_idx, topk_w, stream=None) -> None:
    if shape.T > 0:
        _want(logits, "logits", _F32, shape.T * shape.E)
        _want(topk_idx, "topk_idx", _I32, shape.T * shape.k)
        _want(topk_w, "topk_w", _F32, shape.T * shape.k)
    _check(lib().moe_route(ctypes.byref(shape), _ptr(logits), int(bool(renorm)), _ptr(topk_idx), _ptr(topk_w),
                           _stream(stream)), "moe_route")


def moe_route_bwd(shape, logits, topk_idx, topk_w, d_topk_w, renorm, d_logits, stream=None) -> None:
    if shape.T > 0:
        for t, n, dt, cnt in ((logits, "logits", _F32, shape.T * shape.E),
                              (topk_idx, "topk_idx", _I32, shape.T * shape.k),
                              (topk_w, "topk_w", _F32, shape.T * shape.k),
                              (d_topk_w, "d_topk_w", _F32, shape.T * shape.k),
                              (d_logits, "d_logits", _F32, shape.T * shape.E)):
            _want(t, n, dt, cnt)
    _check(lib().moe_route_bwd(ctypes.byref(shape), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(d_topk_w),
                               int(bool(renorm)), _ptr(d_logits), _stream(stream)), "moe_route_bwd")


def moe_read_status(ws, stream=None) -> int:
    out = ctypes.c_int32()
    _check(lib().moe_read_status(_ptr(ws), ctypes.byref(out), _stream(stream)), "moe_read_status")
    return out.value


def moe_set_kernel_timing(enable: bool) -> None:
    _check(lib().moe_set_kernel_timing(1 if enable else 0), "moe_set_kernel_timing")


def moe_kernel_timing_collect(max_entries: int = 64) -> dict:
    arr = (moe_kernel_time * max_entries)()
    n = ctypes.c_int32()
    _check(lib().moe_kernel_timing_collect(arr, max_entries, ctypes.byref(n)), "moe_kernel_timing_collect")
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


# ------------------------------------------------------------ buffer plumbing

@dataclasses.dataclass
class LayerBuffers:
    """Device buffers of one layer shape (allocated once with torch). `wq`
    holds the quantized weights of the FP8 precisions (None for bf16)."""
    shape: moe_shape
    fwd_ws: torch.Tensor
    saved: torch.Tensor
    bwd_ws: torch.Tensor
    layout: dict
    wq: torch.Tensor | None = None
    wq_layout: dict | None = None

    @classmethod
    def allocate(cls, shape: moe_shape, device="cuda") -> "LayerBuffers":
        f, s, b = moe_workspace_size(shape)
        mk = lambda n: torch.empty(max(n, 256), dtype=torch.uint8, device=device)  # noqa: E731
        wl = moe_get_wq_layout(shape)
        wq = mk(wl["total"]) if wl["total"] > 0 else None
        return cls(shape, mk(f), mk(s), mk(b), moe_get_saved_layout(shape), wq, wl)

    def saved_view(self, name: str, dtype, count: int) -> torch.Tensor:
        off = self.layout[name]
        esz = torch.empty((), dtype=dtype).element_size()
        return self.saved[off:off + count * esz].view(dtype)


def quantize_weights(buf: LayerBuffers, W13, W2, stream=None) -> None:
    """Refreshes buf.wq from the bf16 weights (no-op for bf16)."""
    if buf.wq is not None:
        moe_quantize_weights(buf.shape, W13, W2, buf.wq, stream)


def forward(buf: LayerBuffers, x, topk_idx, topk_w, W13, W2, y=None, training=True, stream=None):
    """Forward; for FP8 precisions buf.wq must hold quantize_weights of W13, W2."""
    s = buf.shape
    if y is None:
        y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=x.device)
    moe_fwd(s, x, topk_idx, topk_w, W13, W2, buf.wq, y, buf.saved if training else None, buf.fwd_ws, stream)
    return y


def forward_logits(buf: LayerBuffers, x, logits, renorm, topk_idx, topk_w, W13, W2, y=None, training=True,
                   stream=None):
    """Forward with the router fused in: writes topk_idx and topk_w."""
    s = buf.shape
    if y is None:
        y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=x.device)
    moe_fwd_logits(s, x, logits, renorm, topk_idx, topk_w, W13, W2, buf.wq, y, buf.saved if training else None,
                   buf.fwd_ws, stream)
    return y


def backward(buf: LayerBuffers, dy, x, topk_idx, topk_w, W13, W2, grads=None, stream=None):
    s = buf.shape
    if grads is None:
        dev = dy.device
        grads = (torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev),
                 torch.empty((s.T, s.k), dtype=torch.float32, device=dev),
                 torch.empty((s.E, 2 * s.I, s.H), dtype=torch.bfloat16, device=dev),
                 torch.empty((s.E, s.H, s.I), dtype=torch.bfloat16, device=dev))
    dx, dw, dW13, dW2 = grads
    moe_bwd(s, dy, x, topk_idx, topk_w, W13, W2, buf.wq, buf.saved, dx, dw, dW13, dW2, buf.bwd_ws, stream)
    return grads
