"""ctypes binding of libgbb.so with the C entry points' names.

Host calls take numpy arrays; device calls take torch tensors on a ROCm
device and enqueue on torch's current stream of that device.  Every function
only checks Python-side types, passes raw pointers and sizes, and turns a
negative status into GbbError with the library's message.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgbb.so")

GBB_PACK_GIVEN_SZ = 1
_STATUS = {0: "GBB_OK", -1: "GBB_E_ARG", -2: "GBB_E_SHAPE", -3: "GBB_E_BITS", -4: "GBB_E_ALIGN",
           -5: "GBB_E_SPACE", -6: "GBB_E_FORMAT", -7: "GBB_E_DEVICE"}


class GbbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_lock = threading.Lock()

_vp, _sz, _i, _u = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint
_SIGS = {
    "gbb_last_error": (ctypes.c_char_p, []),
    "gbb_version": (_i, []),
    "gbb_packed_bytes": (_sz, [_vp, _i, _i]),
    "gbb_pack_blocks": (_i, [_vp, _i, _i, _vp, _vp, _vp, _u, _vp, _sz]),
    "gbb_check_image": (_i, [_vp, _sz, _i, _i]),
    "gbb_packed_bytes_64x64": (_sz, [_vp, _i, _i]),
    "gbb_pack_blocks_64x64": (_i, [_vp, _i, _i, _vp, _vp, _vp, _u, _vp, _sz]),
    "gbb_gemm_mixed_w_64x64_workspace": (_sz, [_i, _i, _i]),
    "gbb_gemm_mixed_w_64x64": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "gbb_gemm_mixed_w_64x64_path": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _sz, _i, _vp]),
    "gbb_gemm_mixed_w_path_workspace": (_sz, [_i, _i, _i, _i]),
    "gbb_gemm_mixed_w_64x64_path_workspace": (_sz, [_i, _i, _i, _i]),
    "gbb_unpack_codes_64x64": (_i, [_vp, _i, _i, _vp, _vp]),
    "gbb_dequant_64x64": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "gbb_allocate_bits": (_i, [_vp, _i, _i, ctypes.c_double, ctypes.c_double, _vp]),
    "gbb_channel_order": (_i, [_vp, _i, _i, _vp, _vp]),
    "gbb_gemm_mixed_w_workspace": (_sz, [_i, _i, _i]),
    "gbb_gemm_mixed_w": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "gbb_gemm_mixed_w_path": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _sz, _i, _vp]),
    "gbb_gemm_mixed_w_noalloc": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp]),
    "gbb_gemm_mixed_w_batched_workspace": (_sz, [_i, _vp, _vp, _i]),
    "gbb_gemm_mixed_w_batched": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "gbb_graph_create": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "gbb_graph_launch": (_i, [_vp, _vp]),
    "gbb_graph_destroy": (_i, [_vp]),
    "gbb_unpack_codes": (_i, [_vp, _i, _i, _vp, _vp]),
    "gbb_dequant": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "gbb_w48_packed_bytes": (_sz, [_i, _i, _i]),
    "gbb_pack_w48": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp, _vp, _sz]),
    "gbb_quant_act_i8": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
    "gbb_gemm_w48a8": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _vp, _i, _vp]),
    "gbb_gemm_w48a8_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "gbb_gemm_w48a8_split": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _sz, _vp]),
    "gbb_w48_group_acc": (_i, [_vp, _i, _i, _i, _vp, _i, _vp, _i, _vp]),
}
EXPORTS = tuple(_SIGS)


def lib():
    """Load libgbb.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m gemm_block_bit_amd.build")
            so = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(so, name)
                fn.restype = res
                fn.argtypes = args
            _lib = so
    return _lib


def _check(st: int):
    if st != 0:
        raise GbbError(st, lib().gbb_last_error().decode())


def _np_ptr(a: np.ndarray | None):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("array must be C-contiguous")
    return a.ctypes.data


def version() -> int:
    return lib().gbb_version()


# ----------------------------------------------------------------------------
# host packers
# ----------------------------------------------------------------------------
def _as_u16(W: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W)
    if W.dtype == np.float16:
        return W.view(np.uint16)
    if W.dtype == np.uint16:
        return W
    raise TypeError("W must be float16 (or its uint16 bit pattern)")


def packed_bytes(bits: np.ndarray, N: int, K: int, block_cols: int = 128) -> int:
    bits = np.ascontiguousarray(bits, np.uint8)
    size_fn, pack_fn = _block_fns(block_cols)
    n = size_fn(_np_ptr(bits), N, K)
    if n == 0:
        # the packer validates the map first and reports the precise status
        _check(pack_fn(None, N, K, _np_ptr(bits), None, None, 0, None, 0))
        _check(-1)
    return n


def _block_fns(block_cols: int):
    L = lib()
    if block_cols == 128:
        return L.gbb_packed_bytes, L.gbb_pack_blocks
    if block_cols == 64:
        return L.gbb_packed_bytes_64x64, L.gbb_pack_blocks_64x64
    raise ValueError("block_cols must be 128 (64x128 blocks) or 64 (64x64 blocks)")


def allocate_bits(W: np.ndarray, target_bits: float, gamma: float = 0.05) -> np.ndarray:
    """Per-block bitwidths uint8 [N/64][K/128] of mean <= target_bits for fp16
    W [N][K] (host; see gbb_allocate_bits)."""
    Wu = _as_u16(W)
    N, K = Wu.shape
    bits = np.empty((N // 64, K // 128), np.uint8)
    _check(lib().gbb_allocate_bits(_np_ptr(Wu), N, K, float(target_bits), float(gamma), _np_ptr(bits)))
    return bits


def channel_order(W: np.ndarray):
    """(row_order int32 [N], col_order int32 [K]) by descending L1 norm of fp16
    W [N][K] (host; see gbb_channel_order)."""
    Wu = _as_u16(W)
    N, K = Wu.shape
    rows = np.empty(N, np.int32)
    cols = np.empty(K, np.int32)
    _check(lib().gbb_channel_order(_np_ptr(Wu), N, K, _np_ptr(rows), _np_ptr(cols)))
    return rows, cols


def pack_blocks(W: np.ndarray, bits: np.ndarray, scale: np.ndarray | None = None,
                zero: np.ndarray | None = None, block_cols: int = 128):
    """Quantize fp16 W [N][K] with the per-block bitwidth map and pack it
    (64 x block_cols blocks: 128, or 64 for 64x64 blocks).  Returns (image
    uint8, scale fp16 [N][K/block_cols], zero fp16 [N][K/block_cols]).  With
    `scale` and `zero` given they are used instead of min/max."""
    Wu = _as_u16(W)
    N, K = Wu.shape
    bits = np.ascontiguousarray(bits, np.uint8)
    size = packed_bytes(bits, N, K, block_cols)
    _, pack_fn = _block_fns(block_cols)
    G = K // block_cols
    image = np.empty(size, np.uint8)
    flags = 0
    if scale is not None or zero is not None:
        if scale is None or zero is None:
            raise ValueError("give both scale and zero")
        s = np.ascontiguousarray(scale, np.float16).copy()
        z = np.ascontiguousarray(zero, np.float16).copy()
        flags = GBB_PACK_GIVEN_SZ
    else:
        s = np.empty((N, G), np.float16)
        z = np.empty((N, G), np.float16)
    _check(pack_fn(_np_ptr(Wu), N, K, _np_ptr(bits), _np_ptr(s), _np_ptr(z), flags, _np_ptr(image), size))
    return image, s, z


def check_image(image: np.ndarray, N: int, K: int) -> None:
    image = np.ascontiguousarray(image, np.uint8)
    _check(lib().gbb_check_image(_np_ptr(image), image.size, N, K))


def w48_packed_bytes(N: int, K: int, n8: int) -> int:
    n = lib().gbb_w48_packed_bytes(N, K, n8)
    if n == 0:
        raise GbbError(-2 if (N > 0 and K > 0) else -1, lib().gbb_last_error().decode())
    return n


def pack_w48(W: np.ndarray, rows8: np.ndarray):
    """Pack fp16 W [N][K]: rows8 (ascending) 8-bit symmetric, the rest 4-bit
    asymmetric.  Returns (image uint8, scale fp16 [N][G], zero uint8 [N][G])."""
    Wu = _as_u16(W)
    N, K = Wu.shape
    rows8 = np.ascontiguousarray(rows8, np.int32)
    size = w48_packed_bytes(N, K, rows8.size)
    image = np.empty(size, np.uint8)
    s = np.empty((N, K // 128), np.float16)
    z = np.empty((N, K // 128), np.uint8)
    _check(lib().gbb_pack_w48(_np_ptr(Wu), N, K, _np_ptr(rows8) if rows8.size else None, rows8.size,
                              _np_ptr(s), _np_ptr(z), _np_ptr(image), size))
    return image, s, z


# ----------------------------------------------------------------------------
# device calls (torch tensors)
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dev_ptr(t, dtype=None, name="tensor"):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


_ws_cache: dict = {}


def gemm_mixed_w_workspace(N: int, K: int, M: int) -> int:
    return lib().gbb_gemm_mixed_w_workspace(N, K, M)


def _workspace(device, nbytes: int):
    """A zero-initialised device buffer per (device, stream) reused across
    calls; the library leaves its counters zero after every call."""
    torch = _torch()
    if nbytes == 0:
        return None
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def gemm_mixed_w_path(image, N: int, K: int, x, path: int, out=None, workspace=None):
    torch = _torch()
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M][{K}]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    need = lib().gbb_gemm_mixed_w_path_workspace(N, K, M, path)   # 0 when the call needs none
    ws = workspace if workspace is not None else _workspace(x.device, need)
    _check(lib().gbb_gemm_mixed_w_path(
        _dev_ptr(image, torch.uint8, "image"), N, K, _dev_ptr(x, torch.float16, "x"),
        _dev_ptr(y, torch.float16, "y"), M,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        path, _stream(x)))
    return y


def gemm_mixed_w(image, N: int, K: int, x, out=None, workspace=None):
    """y = x . dequant(W)^T (fp16 [M][N]) on torch's current stream."""
    return gemm_mixed_w_path(image, N, K, x, 0, out, workspace)


def gemm_mixed_w_noalloc(image, N: int, K: int, x, out=None):
    """gemm_mixed_w without a workspace: the library's fixed per-device
    scratch array holds the split-K accumulators (calls on one GPU must not
    overlap)."""
    torch = _torch()
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M][{K}]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check(lib().gbb_gemm_mixed_w_noalloc(
        _dev_ptr(image, torch.uint8, "image"), N, K, _dev_ptr(x, torch.float16, "x"),
        _dev_ptr(y, torch.float16, "y"), M, _stream(x)))
    return y


def gemm_mixed_w_batched_workspace(shapes, M: int) -> int:
    n = len(shapes)
    Ns = (ctypes.c_int * n)(*[int(N) for N, _ in shapes])
    Ks = (ctypes.c_int * n)(*[int(K) for _, K in shapes])
    return lib().gbb_gemm_mixed_w_batched_workspace(n, Ns, Ks, M)


class Batched:
    """Independent products (image, N, K, x, y) with one M, run by
    gbb_gemm_mixed_w_batched: one launch for M <= 16.  The pointer arrays are
    built once; launch() enqueues on torch's current stream."""

    def __init__(self, calls, workspace=None):
        torch = _torch()
        if not calls:
            raise ValueError("no calls")
        M = calls[0][3].shape[0]
        for (img, N, K, x, y) in calls:
            if x.dim() != 2 or tuple(x.shape) != (M, K) or tuple(y.shape) != (M, N):
                raise ValueError(f"x must be [{M}][{K}] and y [{M}][{N}]")
        n = len(calls)
        self.M, self.n = M, n
        self._images = (ctypes.c_void_p * n)(*[_dev_ptr(c[0], torch.uint8, "image") for c in calls])
        self._N = (ctypes.c_int * n)(*[c[1] for c in calls])
        self._K = (ctypes.c_int * n)(*[c[2] for c in calls])
        self._x = (ctypes.c_void_p * n)(*[_dev_ptr(c[3], torch.float16, "x") for c in calls])
        self._y = (ctypes.c_void_p * n)(*[_dev_ptr(c[4], torch.float16, "y") for c in calls])
        need = lib().gbb_gemm_mixed_w_batched_workspace(n, self._N, self._K, M)
        dev = calls[0][3].device
        self._ws = workspace if workspace is not None else torch.zeros(max(need, 256), dtype=torch.uint8,
                                                                       device=dev)
        self._calls = list(calls)

    def launch(self):
        torch = _torch()
        _check(lib().gbb_gemm_mixed_w_batched(self.n, self._images, self._N, self._K, self._x, self._y, self.M,
                                              self._ws.data_ptr(), self._ws.numel(),
                                              torch.cuda.current_stream(self._ws.device).cuda_stream))


class Graph:
    """gemm_mixed_w calls captured into one HIP graph (gbb_graph_create) and
    replayed by launch().  calls: (image, N, K, x, y) with every x [M][K] and
    y [M][N] on one device and one M.  The tensors are kept referenced here
    and must keep their storage and shapes; the inputs are read and the
    outputs written at each launch."""

    def __init__(self, calls, workspace=None):
        torch = _torch()
        if not calls:
            raise ValueError("no calls")
        M = calls[0][3].shape[0]
        for (img, N, K, x, y) in calls:
            if x.dim() != 2 or tuple(x.shape) != (M, K) or tuple(y.shape) != (M, N):
                raise ValueError(f"x must be [{M}][{K}] and y [{M}][{N}]")
        need = max(gemm_mixed_w_workspace(N, K, M) for (_, N, K, _, _) in calls)
        dev = calls[0][3].device
        self._ws = workspace if workspace is not None else torch.zeros(max(need, 256), dtype=torch.uint8,
                                                                       device=dev)
        n = len(calls)
        images = (ctypes.c_void_p * n)(*[_dev_ptr(c[0], torch.uint8, "image") for c in calls])
        Ns = (ctypes.c_int * n)(*[c[1] for c in calls])
        Ks = (ctypes.c_int * n)(*[c[2] for c in calls])
        xs = (ctypes.c_void_p * n)(*[_dev_ptr(c[3], torch.float16, "x") for c in calls])
        ys = (ctypes.c_void_p * n)(*[_dev_ptr(c[4], torch.float16, "y") for c in calls])
        out = ctypes.c_void_p()
        self._g = None
        _check(lib().gbb_graph_create(n, images, Ns, Ks, xs, ys, M, self._ws.data_ptr(), self._ws.numel(),
                                      ctypes.byref(out)))
        self._g = out
        self._calls = list(calls)

    def launch(self):
        """Replay on torch's current stream of the calls' device."""
        torch = _torch()
        _check(lib().gbb_graph_launch(self._g, torch.cuda.current_stream(self._ws.device).cuda_stream))

    def close(self):
        if self._g is not None:
            g, self._g = self._g, None
            _check(lib().gbb_graph_destroy(g))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def unpack_codes(image, N: int, K: int, block_cols: int = 128):
    torch = _torch()
    q = torch.empty((N, K), dtype=torch.uint8, device=image.device)
    fn = lib().gbb_unpack_codes if block_cols == 128 else lib().gbb_unpack_codes_64x64
    _check(fn(_dev_ptr(image, torch.uint8, "image"), N, K, q.data_ptr(), _stream(image)))
    return q


def dequant(image, N: int, K: int, block_cols: int = 128):
    """(w32 fp32 [N][K] = (q - z) * s, w16 = its fp16 rounding)."""
    torch = _torch()
    w32 = torch.empty((N, K), dtype=torch.float32, device=image.device)
    w16 = torch.empty((N, K), dtype=torch.float16, device=image.device)
    fn = lib().gbb_dequant if block_cols == 128 else lib().gbb_dequant_64x64
    _check(fn(_dev_ptr(image, torch.uint8, "image"), N, K, w32.data_ptr(), w16.data_ptr(), _stream(image)))
    return w32, w16


def gemm_mixed_w_64x64_workspace(N: int, K: int, M: int) -> int:
    return lib().gbb_gemm_mixed_w_64x64_workspace(N, K, M)


def gemm_mixed_w_64x64_path(image, N: int, K: int, x, path: int, out=None, workspace=None):
    """y = x . dequant(W)^T over a 64x64-block image (fp16 [M][N]); path 0
    the library's choice, 1 the decode kernel (M <= 32), 2 the prefill
    kernel."""
    torch = _torch()
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M][{K}]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    need = lib().gbb_gemm_mixed_w_64x64_path_workspace(N, K, M, path)
    ws = workspace if workspace is not None else _workspace(x.device, need)
    _check(lib().gbb_gemm_mixed_w_64x64_path(
        _dev_ptr(image, torch.uint8, "image"), N, K, _dev_ptr(x, torch.float16, "x"),
        _dev_ptr(y, torch.float16, "y"), M, ws.data_ptr() if ws is not None else None,
        ws.numel() if ws is not None else 0, path, _stream(x)))
    return y


def gemm_mixed_w_64x64(image, N: int, K: int, x, out=None, workspace=None):
    """y = x . dequant(W)^T over a 64x64-block image (fp16 [M][N])."""
    return gemm_mixed_w_64x64_path(image, N, K, x, 0, out, workspace)


def quant_act_i8(x, ga: int | None = None):
    """int8 symmetric activations: (xq int8 [M][K], xs fp16 [M] or [M][K/128])."""
    torch = _torch()
    M, K = x.shape
    ga = K if ga is None else ga
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty((M,) if ga == K else (M, K // 128), dtype=torch.float16, device=x.device)
    _check(lib().gbb_quant_act_i8(_dev_ptr(x, torch.float16, "x"), M, K, ga, xq.data_ptr(), xs.data_ptr(),
                                  _stream(x)))
    return xq, xs


def gemm_w48a8_workspace(N: int, K: int, n8: int, M: int, ga: int | None = None) -> int:
    return lib().gbb_gemm_w48a8_workspace(N, K, n8, M, K if ga is None else ga)


def gemm_w48a8(image, N: int, K: int, n8: int, xq, xs, ga: int | None = None, out=None, workspace=None,
               split: bool = True):
    """y = dequant(xq) . dequant(W)^T (fp16 [M][N]) on torch's current
    stream.  split: gbb_gemm_w48a8_split over `workspace` (default: the
    binding's per-stream buffer), else gbb_gemm_w48a8."""
    torch = _torch()
    M = xq.shape[0]
    ga = K if ga is None else ga
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=xq.device)
    args = (_dev_ptr(image, torch.uint8, "image"), N, K, n8, _dev_ptr(xq, torch.int8, "xq"),
            _dev_ptr(xs, torch.float16, "xs"), ga, _dev_ptr(y, torch.float16, "y"), M)
    if not split:
        _check(lib().gbb_gemm_w48a8(*args, _stream(xq)))
        return y
    ws = workspace if workspace is not None else _workspace(xq.device, gemm_w48a8_workspace(N, K, n8, M, ga))
    _check(lib().gbb_gemm_w48a8_split(*args, ws.data_ptr() if ws is not None else None,
                                      ws.numel() if ws is not None else 0, _stream(xq)))
    return y


def w48_group_acc(image, N: int, K: int, n8: int, xq, ga: int | None = None):
    """int32 [M][N][K/128] exact group sums xq . (q - z) from the kernel that
    gbb_gemm_w48a8 runs for this M and ga (K: per-token scales, or 128)."""
    torch = _torch()
    M = xq.shape[0]
    ga = K if ga is None else ga
    acc = torch.empty((M, N, K // 128), dtype=torch.int32, device=xq.device)
    _check(lib().gbb_w48_group_acc(_dev_ptr(image, torch.uint8, "image"), N, K, n8,
                                   _dev_ptr(xq, torch.int8, "xq"), ga, acc.data_ptr(), M, _stream(xq)))
    return acc
