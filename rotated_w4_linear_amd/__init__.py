"""Python binding of the MI355X (gfx950) rotated W4G128 linear library.

Thin ctypes marshalling over ``libparo.so`` (C ABI in ``include/paro.h``):
torch tensors are passed as device pointers plus the current HIP stream, and
every step of the hot path runs in the library's HIP kernels. There is no
fallback: if the library is missing or no GPU is visible the calls raise.

Names follow the C ABI: ``paro_device_init``, ``paro_rotation_create`` / ``Rotation``,
``paro_rotate``, ``paro_quantize_weights``, ``paro_w4_linear``,
``paro_w4_linear_workspace_size``, ``paro_w4_linear_noalloc``, ``paro_rotation_backward``,
``paro_rotation_backward_workspace_size``, ``paro_layer_loss``,
``paro_layer_loss_workspace_size``, ``paro_pairs_random``, ``paro_pairs_by_gap``,
``paro_sparsify_angles``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libparo.so")

PARO_OK = 0
STATUS = {
    0: "PARO_OK", -1: "PARO_ERR_NULL", -2: "PARO_ERR_SHAPE", -3: "PARO_ERR_PAIRING",
    -4: "PARO_ERR_VALUE", -5: "PARO_ERR_ALIGN", -6: "PARO_ERR_UNSUPPORTED",
    -7: "PARO_ERR_WORKSPACE", -8: "PARO_ERR_HIP",
}

_lib = None


class ParoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libparo.so (built by ``rotated_w4_linear_amd.build``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rotated_w4_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_i32, vp, c_size = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.paro_status_string.restype = ctypes.c_char_p
    lib.paro_status_string.argtypes = [ctypes.c_int]
    lib.paro_last_error.restype = ctypes.c_char_p
    lib.paro_last_error.argtypes = []
    lib.paro_device_init.restype = ctypes.c_int
    lib.paro_device_init.argtypes = []
    lib.paro_rotation_create.restype = ctypes.c_int
    lib.paro_rotation_create.argtypes = [c_i64, c_i32, c_i32, vp, vp, vp, ctypes.POINTER(vp)]
    lib.paro_rotation_destroy.restype = None
    lib.paro_rotation_destroy.argtypes = [vp]
    lib.paro_rotation_info.restype = ctypes.c_int
    lib.paro_rotation_info.argtypes = [vp, ctypes.POINTER(c_i64), ctypes.POINTER(c_i32),
                                       ctypes.POINTER(c_i32)]
    lib.paro_rotate.restype = ctypes.c_int
    lib.paro_rotate.argtypes = [vp, vp, vp, c_i64, vp]
    lib.paro_quantize_weights.restype = ctypes.c_int
    lib.paro_quantize_weights.argtypes = [vp, vp, c_i64, c_i64, c_i32, vp, vp, vp, vp]
    lib.paro_w4_linear_workspace_size.restype = c_size
    lib.paro_w4_linear_workspace_size.argtypes = [vp, c_i64, c_i64, c_i64]
    lib.paro_w4_linear.restype = ctypes.c_int
    lib.paro_w4_linear.argtypes = [vp, vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_i32, vp,
                                   c_size, vp]
    lib.paro_w4_linear_noalloc.restype = ctypes.c_int
    lib.paro_w4_linear_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_i32,
                                           vp]
    lib.paro_rotation_backward_workspace_size.restype = c_size
    lib.paro_rotation_backward_workspace_size.argtypes = [vp, c_i64]
    lib.paro_rotation_backward.restype = ctypes.c_int
    lib.paro_rotation_backward.argtypes = [vp, c_i32, vp, vp, vp, vp, vp, c_i64, vp, c_size, vp]
    lib.paro_layer_loss_workspace_size.restype = c_size
    lib.paro_layer_loss_workspace_size.argtypes = [vp, c_i64, c_i64, c_i64, c_i32]
    lib.paro_layer_loss.restype = ctypes.c_int
    lib.paro_layer_loss.argtypes = [vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_i32, vp, vp, vp,
                                    vp, c_size, vp]
    lib.paro_pairs_random.restype = ctypes.c_int
    lib.paro_pairs_random.argtypes = [c_i64, c_i32, c_i32, ctypes.c_uint64, vp]
    lib.paro_pairs_by_gap.restype = ctypes.c_int
    lib.paro_pairs_by_gap.argtypes = [c_i64, c_i32, c_i32, vp, vp]
    lib.paro_sparsify_angles.restype = ctypes.c_int
    lib.paro_sparsify_angles.argtypes = [c_i64, c_i32, vp, c_i64, vp]
    lib.paro_stream_copy.restype = ctypes.c_int
    lib.paro_stream_copy.argtypes = [vp, vp, c_size, c_i32, vp]
    lib.paro_mfma_loop.restype = ctypes.c_int
    lib.paro_mfma_loop.argtypes = [vp, c_i64, vp, c_i32, c_i32, vp]
    lib.paro_rotation_plan_host.restype = ctypes.c_int
    lib.paro_rotation_plan_host.argtypes = [c_i64, c_i32, c_i32, vp, vp, vp, vp, c_size,
                                            ctypes.POINTER(c_size), ctypes.POINTER(c_i32)]
    _lib = lib
    return lib


def _check(status: int):
    if status != PARO_OK:
        raise ParoError(status, load_library().paro_last_error().decode())


def _host_arrays(pairs, theta, alpha):
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32))
    theta = np.ascontiguousarray(np.asarray(theta, dtype=np.float32))
    alpha = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32))
    return pairs, theta, alpha


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dptr(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a ROCm device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def paro_device_init():
    """Per-device set-up of the current device (``paro_device_init``)."""
    _check(load_library().paro_device_init())


class Rotation:
    """``paro_rotation_create`` / ``paro_rotation_destroy`` for one layer's (pairs, theta, alpha)."""

    def __init__(self, pairs, theta, alpha, group: int):
        lib = load_library()
        pairs, theta, alpha = _host_arrays(pairs, theta, alpha)
        self.d = int(alpha.shape[0])
        self.K = int(pairs.shape[0]) if pairs.ndim == 3 else 0
        self.group = int(group)
        h = ctypes.c_void_p()
        _check(lib.paro_rotation_create(self.d, self.group, self.K, _ptr(pairs), _ptr(theta),
                                        _ptr(alpha), ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load_library().paro_rotation_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


paro_rotation_create = Rotation


def _handle(r: Optional[Rotation]):
    return r.handle if r is not None else None


def paro_rotate(r: Rotation, x, y=None, stream=None):
    """X' = X T^-1 row by row (fp16 [M][d] -> fp16 [M][d]); ``y`` may be ``x``."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    _check(load_library().paro_rotate(r.handle, _dptr(x, "x", torch.float16),
                                      _dptr(y, "y", torch.float16), int(x.shape[0]),
                                      _stream(stream)))
    return y


def paro_quantize_weights(r: Optional[Rotation], w, group: int = 128, stream=None):
    """Q(T W) (or Q(W) when ``r`` is None): returns (qweight u8 [N][d/2], scales fp16, zeros u8)."""
    import torch
    N, d = w.shape
    qweight = torch.empty((N, d // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, d // group), dtype=torch.float16, device=w.device)
    zeros = torch.empty((N, d // group), dtype=torch.uint8, device=w.device)
    _check(load_library().paro_quantize_weights(
        _handle(r), _dptr(w, "w", torch.float16), N, d, group, _dptr(qweight, "qweight"),
        _dptr(scales, "scales"), _dptr(zeros, "zeros"), _stream(stream)))
    return qweight, scales, zeros


def paro_w4_linear_workspace_size(r: Optional[Rotation], M: int, N: int, d: int) -> int:
    return int(load_library().paro_w4_linear_workspace_size(_handle(r), M, N, d))


def new_workspace(r: Optional[Rotation], M: int, N: int, d: int, device="cuda"):
    """A zero-filled workspace for paro_w4_linear (None when none is needed)."""
    import torch
    need = paro_w4_linear_workspace_size(r, M, N, d)
    return torch.zeros(need, dtype=torch.uint8, device=device) if need else None


def paro_w4_linear(r: Optional[Rotation], x, qweight, scales, zeros, bias=None, y=None,
                   group: int = 128, workspace=None, stream=None):
    """Y = rot(X) dequant(W)^T + b (fp16 [M][N]); rot is the identity when ``r`` is None."""
    import torch
    M, d = x.shape
    N = qweight.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = new_workspace(r, M, N, d, x.device)
    ws_ptr = _dptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().paro_w4_linear(
        _handle(r), _dptr(x, "x", torch.float16), _dptr(qweight, "qweight", torch.uint8),
        _dptr(scales, "scales", torch.float16), _dptr(zeros, "zeros", torch.uint8),
        _dptr(bias, "bias", torch.float16) if bias is not None else None,
        _dptr(y, "y", torch.float16), M, N, d, group, ws_ptr, ws_bytes, _stream(stream)))
    return y


def paro_w4_linear_noalloc(r: Optional[Rotation], x, qweight, scales, zeros, y, bias=None,
                           group: int = 128, stream=None):
    """``paro_w4_linear`` on the library's static scratch: ``y`` (fp16 [M][N])
    is written in place and nothing is allocated."""
    import torch
    M, d = x.shape
    N = qweight.shape[0]
    _check(load_library().paro_w4_linear_noalloc(
        _handle(r), _dptr(x, "x", torch.float16), _dptr(qweight, "qweight", torch.uint8),
        _dptr(scales, "scales", torch.float16), _dptr(zeros, "zeros", torch.uint8),
        _dptr(bias, "bias", torch.float16) if bias is not None else None,
        _dptr(y, "y", torch.float16), M, N, d, group, _stream(stream)))
    return y


SIDES = {"activation": 0, "weight": 1}


def paro_rotation_backward_workspace_size(r: Rotation, M: int) -> int:
    return int(load_library().paro_rotation_backward_workspace_size(r.handle, M))


def paro_rotation_backward(r: Rotation, x, gy, side: str = "activation", gx=None,
                           want_gx: bool = True, workspace=None, stream=None):
    """Gradients of the transform: returns (gx fp32 [M][d] or None, dtheta fp32
    [K][d/2], dalpha fp32 [d]) for x fp16 [M][d] and gy = dL/d(output) fp32."""
    import torch
    M, d = x.shape
    info_K = r.K
    if gx is None and want_gx:
        gx = torch.empty((M, d), dtype=torch.float32, device=x.device)
    dtheta = torch.empty((info_K, d // 2), dtype=torch.float32, device=x.device)
    dalpha = torch.empty((d,), dtype=torch.float32, device=x.device)
    if workspace is None:
        need = paro_rotation_backward_workspace_size(r, M)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    ws_ptr = _dptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().paro_rotation_backward(
        r.handle, SIDES[side], _dptr(x, "x", torch.float16), _dptr(gy, "gy", torch.float32),
        _dptr(gx, "gx", torch.float32) if gx is not None else None,
        _dptr(dtheta, "dtheta", torch.float32) if info_K else None,
        _dptr(dalpha, "dalpha", torch.float32), M, ws_ptr, ws_bytes, _stream(stream)))
    return gx, dtheta, dalpha


def paro_layer_loss(r: Rotation, x, w, qweight, scales, zeros, gradients: bool = True,
                    workspace=None, stream=None):
    """Layer-wise output loss sum (Y_q - X W^T)^2 (fp32 device scalar) and, with
    ``gradients``, its straight-through dtheta [K][d/2] and dalpha [d]."""
    import torch
    M, d = x.shape
    N = w.shape[0]
    dev_ = x.device
    loss = torch.empty((1,), dtype=torch.float32, device=dev_)
    dth = torch.empty((r.K, d // 2), dtype=torch.float32, device=dev_) if gradients else None
    dal = torch.empty((d,), dtype=torch.float32, device=dev_) if gradients else None
    if workspace is None:
        need = int(load_library().paro_layer_loss_workspace_size(r.handle, M, N, d, int(gradients)))
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev_) if need else None
    ws_ptr = _dptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().paro_layer_loss(
        r.handle, _dptr(x, "x", torch.float16), _dptr(w, "w", torch.float16),
        _dptr(qweight, "qweight", torch.uint8), _dptr(scales, "scales", torch.float16),
        _dptr(zeros, "zeros", torch.uint8), M, N, d, r.group, _dptr(loss, "loss", torch.float32),
        _dptr(dth, "dtheta", torch.float32) if (gradients and r.K) else None,
        _dptr(dal, "dalpha", torch.float32) if gradients else None, ws_ptr, ws_bytes,
        _stream(stream)))
    return loss, dth, dal


def paro_rotation_plan_host(pairs, theta, alpha, group: int) -> Tuple[np.ndarray, dict]:
    """Host-only schedule image (what paro_rotation_create uploads) and its layout."""
    lib = load_library()
    pairs, theta, alpha = _host_arrays(pairs, theta, alpha)
    d = int(alpha.shape[0])
    K = int(pairs.shape[0]) if pairs.ndim == 3 else 0
    need = ctypes.c_size_t()
    lay = (ctypes.c_int32 * 5)()
    _check(lib.paro_rotation_plan_host(d, group, K, _ptr(pairs), _ptr(theta), _ptr(alpha), None,
                                       0, ctypes.byref(need), lay))
    img = np.zeros(need.value // 4, dtype=np.uint32)
    _check(lib.paro_rotation_plan_host(d, group, K, _ptr(pairs), _ptr(theta), _ptr(alpha),
                                       img.ctypes.data_as(ctypes.c_void_p), need.value,
                                       ctypes.byref(need), lay))
    return img, {"seg_ch": lay[0], "ppl": lay[1], "words": lay[2], "fast": bool(lay[3]),
                 "stages": lay[4]}


def paro_pairs_random(d: int, group: int, K: int, seed: int) -> np.ndarray:
    """Random pairs with de-duplication across stages: int32 [K][d/2][2]."""
    out = np.zeros((K, d // 2, 2), dtype=np.int32)
    _check(load_library().paro_pairs_random(d, group, K, ctypes.c_uint64(seed & (2 ** 64 - 1)),
                                            _ptr(out)))
    return out


def paro_pairs_by_gap(score, group: int, K: int) -> np.ndarray:
    """Pairs of strongly differing channels by per-channel ``score``: int32 [K][d/2][2]."""
    score = np.ascontiguousarray(np.asarray(score, dtype=np.float32))
    d = int(score.shape[0])
    out = np.zeros((K, d // 2, 2), dtype=np.int32)
    _check(load_library().paro_pairs_by_gap(d, group, K, _ptr(score), _ptr(out)))
    return out


def paro_sparsify_angles(theta, n_keep: int) -> np.ndarray:
    """The ``n_keep`` largest-|theta| pairs keep their angle, the rest get 0."""
    theta = np.ascontiguousarray(np.asarray(theta, dtype=np.float32))
    K, half = theta.shape
    out = np.zeros_like(theta)
    _check(load_library().paro_sparsify_angles(2 * half, K, _ptr(theta), int(n_keep), _ptr(out)))
    return out


def paro_stream_copy(src, dst, blocks: int = 8192, stream=None):
    """Plain device copy of ``src`` into ``dst`` (same byte size): the
    measured HBM ceiling the memory-bound kernels are reported against."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size")
    _check(load_library().paro_stream_copy(_dptr(src, "src"), _dptr(dst, "dst"), nbytes, int(blocks),
                                           _stream(stream)))
    return dst


def paro_mfma_loop(src, out, blocks: int, iters: int, stream=None):
    """fp16 matrix-core loop on operands read from ``src`` (fp16, a multiple of
    8 elements); ``out`` holds blocks * 256 floats: the measured matrix-core
    ceiling the prefill linear is reported against."""
    import torch
    if src.numel() % 8:
        raise ValueError("src must hold a multiple of 8 elements")
    if out.numel() < int(blocks) * 256:
        raise ValueError("out must hold blocks * 256 floats")
    _check(load_library().paro_mfma_loop(_dptr(src, "src", torch.float16), src.numel(),
                                         _dptr(out, "out", torch.float32), int(blocks), int(iters),
                                         _stream(stream)))
    return out
