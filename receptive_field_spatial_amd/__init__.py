"""WBMM (Windowed Batch Matrix Multiplication) for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libwbmm.so`` (declared in ``include/wbmm.h``). Each
function here has the C entry point's name and only marshals arguments: PyTorch supplies device
memory and the current stream, every step of the operator runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing or cannot load, calls raise ``WbmmError``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

__all__ = [
    "WbmmError", "lib_path", "load_library", "abi_version",
    "wbmm_build_index", "wbmm_build_matrix", "wbmm_fold_hier",
    "wbmm_forward", "wbmm_forward_workspace_bytes",
    "wbmm_backward", "wbmm_backward_workspace_bytes", "wbmm_set_launch_events",
    "wbmm_forward_hier", "wbmm_forward_hier_workspace_bytes",
    "wbmm_backward_hier", "wbmm_backward_hier_workspace_bytes", "wbmm_dwconv_forward",
    "wbmm_forward_shifted", "wbmm_forward_shifted_workspace_bytes", "wbmm_backward_shifted",
    "wbmm_backward_shifted_workspace_bytes", "wbmm_probe_mfma", "wbmm_backward_bf16",
    "wbmm_backward_bf16_workspace_bytes", "wbmm_backward_noalloc", "WBMM_NOALLOC_SCRATCH_BYTES",
    "WBMM_OK", "WBMM_E_INVALID", "WBMM_E_UNSUPPORTED", "WBMM_E_WORKSPACE", "WBMM_E_HIP",
]

WBMM_OK, WBMM_E_INVALID, WBMM_E_UNSUPPORTED, WBMM_E_WORKSPACE, WBMM_E_HIP = range(5)
WBMM_F32, WBMM_BF16 = 0, 1
WBMM_NCHW, WBMM_NHWC = 0, 1
WBMM_NOALLOC_SCRATCH_BYTES = 32 << 20  # the library's fixed scratch for wbmm_backward_noalloc

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()


class WbmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"wbmm status {status}: {message}")
        self.status = status


def lib_path() -> str:
    return os.path.join(_PKG_DIR, "libwbmm.so")


def _declare(lib):
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    sigs = {
        "wbmm_abi_version": (c_int, []),
        "wbmm_last_error": (ctypes.c_char_p, []),
        "wbmm_build_index": (c_int, [c_int, vp, vp]),
        "wbmm_build_matrix": (c_int, [vp, c_int, c_int, c_int, vp, vp]),
        "wbmm_fold_hier": (c_int, [vp, vp, c_int, c_int, c_int, c_int, vp, vp]),
        "wbmm_forward_workspace_bytes": (c_size, [c_int] * 8),
        "wbmm_forward": (c_int, [c_int] * 8 + [vp] * 7 + [c_size, vp]),
        "wbmm_backward_workspace_bytes": (c_size, [c_int] * 7),
        "wbmm_backward": (c_int, [c_int] * 6 + [vp] * 10 + [c_size, vp]),
        "wbmm_set_launch_events": (c_int, [vp, vp]),
        "wbmm_forward_hier_workspace_bytes": (c_size, [c_int] * 9),
        "wbmm_forward_hier": (c_int, [c_int] * 7 + [vp] * 7 + [c_size, vp]),
        "wbmm_backward_hier_workspace_bytes": (c_size, [c_int] * 8),
        "wbmm_backward_hier": (c_int, [c_int] * 7 + [vp] * 11 + [c_size, vp]),
        "wbmm_dwconv_forward": (c_int, [c_int] * 5 + [vp] * 4),
        "wbmm_probe_mfma_flops": (ctypes.c_double, [c_int] * 3),
        "wbmm_backward_bf16_workspace_bytes": (c_size, [c_int] * 7),
        "wbmm_backward_bf16": (c_int, [c_int] * 6 + [vp] * 9 + [c_size, vp]),
        "wbmm_probe_mfma": (c_int, [c_int] * 3 + [vp, vp]),
        "wbmm_forward_shifted_workspace_bytes": (c_size, [c_int] * 10),
        "wbmm_forward_shifted": (c_int, [c_int] * 10 + [vp] * 7 + [c_size, vp]),
        "wbmm_backward_shifted_workspace_bytes": (c_size, [c_int] * 9),
        "wbmm_backward_shifted": (c_int, [c_int] * 8 + [vp] * 10 + [c_size, vp]),
        "wbmm_backward_noalloc": (c_int, [c_int] * 6 + [vp] * 10),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load_library(path: Optional[str] = None):
    """Load libwbmm.so (built in-tree by ``receptive_field_spatial_amd.build``)."""
    global _LIB
    with _LOCK:
        if _LIB is None or path is not None:
            p = path or lib_path()
            if not os.path.exists(p):
                raise WbmmError(WBMM_E_UNSUPPORTED,
                                f"{p} is missing: build it with `python -m receptive_field_spatial_amd.build`")
            _LIB = _declare(ctypes.CDLL(p))
        return _LIB


def _lib():
    return _LIB if _LIB is not None else load_library()


def abi_version() -> int:
    return _lib().wbmm_abi_version()


def _check(status: int):
    if status != WBMM_OK:
        raise WbmmError(status, _lib().wbmm_last_error().decode(errors="replace"))


# ----------------------------------------------------------------------------- torch plumbing
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise WbmmError(WBMM_E_INVALID, "tensors must be on the GPU")
    if not t.is_contiguous():
        raise WbmmError(WBMM_E_INVALID, "tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return WBMM_F32
    if dt == torch.bfloat16:
        return WBMM_BF16
    raise WbmmError(WBMM_E_INVALID, f"unsupported dtype {dt}")


def _layout_code(layout: str) -> int:
    if layout.upper() == "NCHW":
        return WBMM_NCHW
    if layout.upper() == "NHWC":
        return WBMM_NHWC
    raise WbmmError(WBMM_E_INVALID, f"unknown layout {layout}")


def _bchw(x, layout: str):
    if x.dim() != 4:
        raise WbmmError(WBMM_E_INVALID, "feature maps are 4-D")
    if _layout_code(layout) == WBMM_NCHW:
        B, C, H, W = x.shape
    else:
        B, H, W, C = x.shape
    return int(B), int(C), int(H), int(W)


# ----------------------------------------------------------------------------- entry points
def wbmm_build_index(w: int, out=None, stream=None):
    """int32 (d, d) relative-position index of one w x w window."""
    torch = _torch()
    d = w * w
    if out is None:
        out = torch.empty((d, d), dtype=torch.int32, device="cuda")
    _check(_lib().wbmm_build_index(int(w), _ptr(out), _stream(stream)))
    return out


def wbmm_build_matrix(T, w: int, out=None, stream=None):
    """Cached matrices M (C, d, d) gathered from the tables T (C, 2w-1, 2w-1)."""
    torch = _torch()
    C = int(T.shape[0])
    d = w * w
    if out is None:
        out = torch.empty((C, d, d), dtype=T.dtype, device=T.device)
    _check(_lib().wbmm_build_matrix(_ptr(T), C, int(w), _dtype_code(T.dtype), _ptr(out),
                                    _stream(stream)))
    return out


def wbmm_fold_hier(M_in, T_sub, w: int, s: int, out=None, stream=None):
    """Fold the s x s sub-window tables T_sub (C, 2s-1, 2s-1) into M_in (C, d, d)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(M_in)
    _check(_lib().wbmm_fold_hier(_ptr(M_in), _ptr(T_sub), int(M_in.shape[0]), int(w), int(s),
                                 _dtype_code(M_in.dtype), _ptr(out), _stream(stream)))
    return out


def wbmm_forward_workspace_bytes(B, C, H, W, w, layout="NCHW", has_mix=False, has_z_save=False) -> int:
    return int(_lib().wbmm_forward_workspace_bytes(B, C, H, W, w, _layout_code(layout),
                                                   int(bool(has_mix)), int(bool(has_z_save))))


def wbmm_forward(x, w: int, T=None, M=None, mix_w=None, *, layout: str = "NCHW", out_dtype=None,
                 y=None, z_save=None, workspace=None, stream=None):
    """Layer forward. Returns y (and z_save, when given, holds the pre-mix output)."""
    return _forward(x, w, None, T, M, mix_w, layout, out_dtype, y, z_save, workspace, stream)


def wbmm_forward_shifted_workspace_bytes(B, C, H, W, w, oy, ox, layout="NCHW", has_mix=False,
                                         has_z_save=False) -> int:
    return int(_lib().wbmm_forward_shifted_workspace_bytes(B, C, H, W, int(w), int(oy), int(ox),
                                                           _layout_code(layout),
                                                           int(bool(has_mix)),
                                                           int(bool(has_z_save))))


def wbmm_forward_shifted(x, w: int, oy: int, ox: int, T=None, M=None, mix_w=None, *,
                         layout: str = "NCHW", out_dtype=None, y=None, z_save=None,
                         workspace=None, stream=None):
    """Layer forward on the window grid offset by (oy, ox) (interleaved windows). Returns y."""
    return _forward(x, w, (int(oy), int(ox)), T, M, mix_w, layout, out_dtype, y, z_save,
                    workspace, stream)


def _forward(x, w, shift, T, M, mix_w, layout, out_dtype, y, z_save, workspace, stream):
    torch = _torch()
    B, C, H, W = _bchw(x, layout)
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    if shift is None:
        need = wbmm_forward_workspace_bytes(B, C, H, W, w, layout, mix_w is not None,
                                            z_save is not None)
    else:
        need = wbmm_forward_shifted_workspace_bytes(B, C, H, W, w, shift[0], shift[1], layout,
                                                    mix_w is not None, z_save is not None)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_layout_code(layout), _dtype_code(x.dtype), _dtype_code(out_dtype), _ptr(x), _ptr(T),
            _ptr(M), _ptr(mix_w), _ptr(z_save), _ptr(y), _ptr(workspace), ws_bytes,
            _stream(stream))
    if shift is None:
        _check(_lib().wbmm_forward(B, C, H, W, int(w), *args))
    else:
        _check(_lib().wbmm_forward_shifted(B, C, H, W, int(w), shift[0], shift[1], *args))
    return y


def wbmm_backward_workspace_bytes(B, C, H, W, w, layout="NCHW", has_mix=False) -> int:
    return int(_lib().wbmm_backward_workspace_bytes(B, C, H, W, w, _layout_code(layout),
                                                    int(bool(has_mix))))


def wbmm_backward(x, dy, w: int, T=None, M=None, mix_w=None, z_saved=None, *, layout: str = "NCHW",
                  dx=True, dT=True, dmix_w=True, workspace=None, stream=None):
    """Layer backward (fp32). Returns (dx, dT, dmix_w); an output passed as False is skipped.

    ``workspace`` (uint8, at least wbmm_backward_workspace_bytes); one is allocated when None.
    """
    return _backward(x, dy, w, None, T, M, mix_w, z_saved, layout, dx, dT, dmix_w, workspace,
                     stream)


def wbmm_backward_noalloc(x, dy, w: int, T=None, M=None, mix_w=None, z_saved=None, *,
                          layout: str = "NCHW", dx=True, dT=True, dmix_w=True, stream=None):
    """wbmm_backward without a workspace: the library's own fixed scratch (one per GPU,
    WBMM_NOALLOC_SCRATCH_BYTES) holds what the backward needs, and the C call allocates nothing.
    Outputs passed as tensors are written in place (pass them all to keep the whole call free of
    allocations); True allocates one here, False skips it. Returns (dx, dT, dmix_w)."""
    torch = _torch()
    B, C, H, W = _bchw(x, layout)
    L = 2 * w - 1
    dev = x.device
    dx_t = torch.empty_like(x) if dx is True else (dx if dx is not False else None)
    dT_t = torch.empty((C, L, L), dtype=torch.float32, device=dev) if dT is True else (dT if dT is not False else None)
    if mix_w is None:
        dW_t = None
    else:
        dW_t = torch.empty((C, 3, 3), dtype=torch.float32, device=dev) if dmix_w is True else (dmix_w if dmix_w is not False else None)
    _check(_lib().wbmm_backward_noalloc(B, C, H, W, int(w), _layout_code(layout), _ptr(x), _ptr(T),
                                        _ptr(M), _ptr(mix_w), _ptr(z_saved), _ptr(dy), _ptr(dx_t),
                                        _ptr(dT_t), _ptr(dW_t), _stream(stream)))
    return dx_t, dT_t, dW_t


def wbmm_backward_shifted_workspace_bytes(B, C, H, W, w, oy, ox, layout="NCHW",
                                          has_mix=False) -> int:
    return int(_lib().wbmm_backward_shifted_workspace_bytes(B, C, H, W, int(w), int(oy), int(ox),
                                                            _layout_code(layout),
                                                            int(bool(has_mix))))


def wbmm_backward_shifted(x, dy, w: int, oy: int, ox: int, T=None, M=None, mix_w=None,
                          z_saved=None, *, layout: str = "NCHW", dx=True, dT=True, dmix_w=True,
                          workspace=None, stream=None):
    """Backward of wbmm_forward_shifted (fp32). Returns (dx, dT, dmix_w)."""
    return _backward(x, dy, w, (int(oy), int(ox)), T, M, mix_w, z_saved, layout, dx, dT, dmix_w,
                     workspace, stream)


def _backward(x, dy, w, shift, T, M, mix_w, z_saved, layout, dx, dT, dmix_w, workspace, stream):
    torch = _torch()
    B, C, H, W = _bchw(x, layout)
    L = 2 * w - 1
    dev = x.device
    dx_t = torch.empty_like(x) if dx is True else (dx if dx is not False else None)
    dT_t = torch.empty((C, L, L), dtype=torch.float32, device=dev) if dT is True else (dT if dT is not False else None)
    if mix_w is None:
        dW_t = None
    else:
        dW_t = torch.empty((C, 3, 3), dtype=torch.float32, device=dev) if dmix_w is True else (dmix_w if dmix_w is not False else None)
    if shift is None:
        need = wbmm_backward_workspace_bytes(B, C, H, W, w, layout, mix_w is not None)
    else:
        need = wbmm_backward_shifted_workspace_bytes(B, C, H, W, w, shift[0], shift[1], layout,
                                                     mix_w is not None)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_layout_code(layout), _ptr(x), _ptr(T), _ptr(M), _ptr(mix_w), _ptr(z_saved), _ptr(dy),
            _ptr(dx_t), _ptr(dT_t), _ptr(dW_t), _ptr(workspace), ws_bytes, _stream(stream))
    if shift is None:
        _check(_lib().wbmm_backward(B, C, H, W, int(w), *args))
    else:
        _check(_lib().wbmm_backward_shifted(B, C, H, W, int(w), shift[0], shift[1], *args))
    return dx_t, dT_t, dW_t


def wbmm_forward_hier_workspace_bytes(B, C, H, W, w, s, layout="NCHW", has_mix=False,
                                      has_z_save=False) -> int:
    return int(_lib().wbmm_forward_hier_workspace_bytes(B, C, H, W, int(w), int(s),
                                                        _layout_code(layout), int(bool(has_mix)),
                                                        int(bool(has_z_save))))


def wbmm_forward_hier(x, w: int, s: int, T, T_sub, mix_w=None, *, layout: str = "NCHW", y=None,
                      z_save=None, workspace=None, stream=None):
    """Layer forward (fp32) with the s x s sub-window tables T_sub (C, 2s-1, 2s-1) folded into
    the matrix (s divides w and s < w; on chip for the quadrants, w = 2s <= 16, otherwise into a
    matrix in the workspace). Returns y (and z_save, when given, holds the pre-mix output)."""
    torch = _torch()
    B, C, H, W = _bchw(x, layout)
    if y is None:
        y = torch.empty_like(x)
    need = wbmm_forward_hier_workspace_bytes(B, C, H, W, w, s, layout, mix_w is not None,
                                             z_save is not None)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().wbmm_forward_hier(B, C, H, W, int(w), int(s), _layout_code(layout), _ptr(x),
                                    _ptr(T), _ptr(T_sub), _ptr(mix_w), _ptr(z_save), _ptr(y),
                                    _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def wbmm_backward_hier_workspace_bytes(B, C, H, W, w, s, layout="NCHW", has_mix=False) -> int:
    return int(_lib().wbmm_backward_hier_workspace_bytes(B, C, H, W, int(w), int(s),
                                                         _layout_code(layout), int(bool(has_mix))))


def wbmm_backward_hier(x, dy, w: int, s: int, T, T_sub, mix_w=None, z_saved=None, *,
                       layout: str = "NCHW", dx=True, dT=True, dT_sub=True, dmix_w=True,
                       workspace=None, stream=None):
    """Backward of wbmm_forward_hier (fp32). Returns (dx, dT, dT_sub, dmix_w); an output passed as
    False is skipped."""
    torch = _torch()
    B, C, H, W = _bchw(x, layout)
    L, Ls = 2 * w - 1, 2 * s - 1
    dev = x.device

    def out(v, shape):
        return torch.empty(shape, dtype=torch.float32, device=dev) if v is True else (v if v is not False else None)

    dx_t = out(dx, tuple(x.shape))
    dT_t = out(dT, (C, L, L))
    dTs_t = out(dT_sub, (C, Ls, Ls))
    dW_t = None if mix_w is None else out(dmix_w, (C, 3, 3))
    need = wbmm_backward_hier_workspace_bytes(B, C, H, W, w, s, layout, mix_w is not None)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().wbmm_backward_hier(B, C, H, W, int(w), int(s), _layout_code(layout), _ptr(x),
                                     _ptr(T), _ptr(T_sub), _ptr(mix_w), _ptr(z_saved), _ptr(dy),
                                     _ptr(dx_t), _ptr(dT_t), _ptr(dTs_t), _ptr(dW_t),
                                     _ptr(workspace), ws_bytes, _stream(stream)))
    return dx_t, dT_t, dTs_t, dW_t


def wbmm_set_launch_events(before, after):
    """Attach two HIP events (raw handles) to the dispatch of the next forward/backward call's
    main kernel: their elapsed time is that kernel's execution."""
    _check(_lib().wbmm_set_launch_events(before, after))


def wbmm_dwconv_forward(x, w_dw, *, y=None, stream=None):
    """k x k depthwise convolution (DW-Std, the pages' comparison operator): fp32 NCHW x
    (B, C, H, W), weights w_dw (C, k, k), zero padding k // 2, stride 1. Returns y."""
    torch = _torch()
    B, C, H, W = _bchw(x, "NCHW")
    k = int(w_dw.shape[-1])
    if tuple(w_dw.shape) != (C, k, k):
        raise WbmmError(WBMM_E_INVALID, f"w_dw must be (C, k, k), got {tuple(w_dw.shape)}")
    if x.dtype != torch.float32 or w_dw.dtype != torch.float32:
        raise WbmmError(WBMM_E_INVALID, "the depthwise convolution is fp32")
    if y is None:
        y = torch.empty_like(x)
    _check(_lib().wbmm_dwconv_forward(B, C, H, W, k, _ptr(x), _ptr(w_dw), _ptr(y),
                                      _stream(stream)))
    return y


def wbmm_probe_mfma(dtype, blocks: int, iters: int, *, out=None, stream=None) -> float:
    """Matrix-core peak probe (measurement aid): launches it and returns the launch's flops.
    dtype: torch.float32 or torch.bfloat16 (the MFMA operand type)."""
    torch = _torch()
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    code = _dtype_code(dtype)
    _check(_lib().wbmm_probe_mfma(code, int(blocks), int(iters), _ptr(out), _stream(stream)))
    return float(_lib().wbmm_probe_mfma_flops(code, int(blocks), int(iters)))


def wbmm_backward_bf16_workspace_bytes(B, C, H, W, w, layout="NCHW", has_mix=False) -> int:
    return int(_lib().wbmm_backward_bf16_workspace_bytes(B, C, H, W, int(w), _layout_code(layout),
                                                         int(bool(has_mix))))


def wbmm_backward_bf16(x, dy, w: int, T, mix_w=None, z_saved=None, *, layout: str = "NCHW",
                       dx=True, dT=True, dmix_w=True, workspace=None, stream=None):
    """Layer backward with bf16 maps (x, dy, z_saved bf16; T bf16). Returns (dx bf16, dT fp32,
    dmix_w fp32); an output passed as False is skipped."""
    torch = _torch()
    B, C, H, W = _bchw(x, layout)
    L = 2 * w - 1
    dev = x.device
    dx_t = torch.empty_like(x) if dx is True else (dx if dx is not False else None)
    dT_t = torch.empty((C, L, L), dtype=torch.float32, device=dev) if dT is True else (dT if dT is not False else None)
    if mix_w is None:
        dW_t = None
    else:
        dW_t = torch.empty((C, 3, 3), dtype=torch.float32, device=dev) if dmix_w is True else (dmix_w if dmix_w is not False else None)
    need = wbmm_backward_bf16_workspace_bytes(B, C, H, W, w, layout, mix_w is not None)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib().wbmm_backward_bf16(B, C, H, W, int(w), _layout_code(layout), _ptr(x), _ptr(T),
                                     _ptr(mix_w),
                                     _ptr(z_saved), _ptr(dy), _ptr(dx_t), _ptr(dT_t), _ptr(dW_t),
                                     _ptr(workspace), ws_bytes, _stream(stream)))
    return dx_t, dT_t, dW_t
