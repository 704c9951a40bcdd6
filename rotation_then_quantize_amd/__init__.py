"""Python binding of librtq, the MI355X (gfx950) rotate-then-quantize linear layer.

Argument marshalling only: every step of the computation runs in librtq's HIP kernels behind the
C ABI declared in ``include/rtq.h``.  torch supplies device memory and the current stream.  There
is no CPU or PyTorch fallback: if ``librtq.so`` is missing, every call raises.

The method (OrbitQuant article, hotelren.com/news/3376620, sections 2.1-2.3): weights are rotated
offline, W' = W Pi^T, and quantised per row; activations are rotated online, x' = Pi x, quantised
per token and multiplied against the quantised weights, where Pi^T Pi = I cancels.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librtq.so")

RTQ_OK, RTQ_ERR_INVALID_ARG, RTQ_ERR_UNSUPPORTED, RTQ_ERR_MISALIGNED, RTQ_ERR_HIP = 0, -1, -2, -3, -4
RTQ_F32, RTQ_BF16, RTQ_I32 = 0, 1, 2
RTQ_INT8, RTQ_CODEBOOK, RTQ_CODEBOOK_I8, RTQ_INT8_TILED = 0, 1, 2, 3
RTQ_CODEBOOK_TILED, RTQ_CODEBOOK_I8_TILED = 4, 5
TILE_ROWS, TILE_K = 256, 64   # the tiled layouts: 256-row tiles, K slices of 64 elements
_CODEBOOK_MODES = (RTQ_CODEBOOK, RTQ_CODEBOOK_I8, RTQ_CODEBOOK_TILED, RTQ_CODEBOOK_I8_TILED)


def tiled_rows(rows: int) -> int:
    """Rows a codes buffer in a tiled layout holds (rows padded to a multiple of 256)."""
    return -(-rows // TILE_ROWS) * TILE_ROWS


def tiled_code_bytes(rows: int, d: int, mode: int, bits: int = 8) -> int:
    """Bytes of a codes buffer in the tiled layout of `mode` (0 for the row-major modes)."""
    if mode in (RTQ_INT8_TILED, RTQ_CODEBOOK_I8_TILED):
        return tiled_rows(rows) * d
    if mode == RTQ_CODEBOOK_TILED:
        return tiled_rows(rows) * d * bits // 8
    return 0

EXPORTS = ("rtq_rpbh_make", "rtq_lloyd_max", "rtq_rpbh_rotate", "rtq_quantize_rows", "rtq_qgemm",
           "rtq_qgemm_ws", "rtq_qgemm_workspace", "rtq_rotated_qlinear", "rtq_rotated_qlinear_workspace",
           "rtq_quantize_rows_asym", "rtq_qgemm_asym", "rtq_rotated_qlinear_asym",
           "rtq_rotated_qlinear_asym_workspace", "rtq_rotated_qlinear_noalloc", "rtq_last_error")

NOALLOC_SCRATCH_BYTES = 96 << 20   # RTQ_NOALLOC_SCRATCH_BYTES


class RtqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"librtq status {status}: {message}")
        self.status = status


class _Rpbh(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("h", ctypes.c_int32), ("perm", ctypes.c_void_p), ("signs", ctypes.c_void_p)]


class _Codebook(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("centroids", ctypes.c_void_p), ("boundaries", ctypes.c_void_p)]


_lib = None


def load_library():
    """Load librtq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           f"(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_float, ctypes.c_size_t)
    R = ctypes.POINTER(_Rpbh)
    C = ctypes.POINTER(_Codebook)
    lib.rtq_rpbh_make.argtypes = [u64, i32, i32, vp, vp]
    lib.rtq_lloyd_max.argtypes = [i32, i32, vp, vp]
    lib.rtq_rpbh_rotate.argtypes = [vp, i32, vp, i32, i64, R, i32, vp]
    lib.rtq_quantize_rows.argtypes = [vp, i32, i64, i32, R, i32, C, f32, vp, vp, i32, vp]
    lib.rtq_qgemm.argtypes = [vp, vp, i64, vp, vp, i32, i64, i32, i32, C, C, vp, i32, vp]
    lib.rtq_qgemm_ws.argtypes = [vp, vp, i64, vp, vp, i32, i64, i32, i32, C, C, vp, i32, vp, sz, vp]
    lib.rtq_qgemm_workspace.argtypes = []
    lib.rtq_qgemm_workspace.restype = sz
    lib.rtq_rotated_qlinear.argtypes = [vp, i32, i64, R, vp, vp, i32, i64, i32, C, C, vp, i32, vp, sz, vp]
    lib.rtq_rotated_qlinear_noalloc.argtypes = [vp, i32, i64, R, vp, vp, i32, i64, i32, C, C, vp, i32, vp]
    lib.rtq_rotated_qlinear_workspace.argtypes = [i64, i32, i32, i32]
    lib.rtq_rotated_qlinear_workspace.restype = sz
    lib.rtq_quantize_rows_asym.argtypes = [vp, i32, i64, i32, R, vp, vp, i32, vp, vp, vp]
    lib.rtq_qgemm_asym.argtypes = [vp, vp, vp, vp, i64, vp, vp, i32, vp, vp, i64, i32, vp, i32, vp, sz, vp]
    lib.rtq_rotated_qlinear_asym.argtypes = [vp, i32, i64, R, vp, vp, i32, vp, vp, i64, vp, i32, vp, sz, vp]
    lib.rtq_rotated_qlinear_asym_workspace.argtypes = [i64, i32]
    lib.rtq_rotated_qlinear_asym_workspace.restype = sz
    lib.rtq_last_error.argtypes = []
    lib.rtq_last_error.restype = ctypes.c_char_p
    for name in ("rtq_rpbh_make", "rtq_lloyd_max", "rtq_rpbh_rotate", "rtq_quantize_rows", "rtq_qgemm",
                 "rtq_qgemm_ws", "rtq_rotated_qlinear", "rtq_quantize_rows_asym", "rtq_qgemm_asym",
                 "rtq_rotated_qlinear_asym", "rtq_rotated_qlinear_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().rtq_last_error().decode()


def _check(status: int):
    if status != RTQ_OK:
        raise RtqError(status, last_error())


# ------------------------------------------------------------------ host helpers

def rpbh_make(seed: int, d: int, h: int = 64):
    """Seeded RPBH descriptor as host arrays (perm int32[d], signs int8[d])."""
    perm = np.empty(d, np.int32)
    signs = np.empty(d, np.int8)
    _check(load_library().rtq_rpbh_make(seed & 0xFFFFFFFFFFFFFFFF, d, h, perm.ctypes.data, signs.ctypes.data))
    return perm, signs


def lloyd_max(d: int, bits: int):
    """Lloyd-Max codebook for N(0, 1/d): (centroids fp32[2^bits], boundaries fp32[2^bits-1])."""
    c = np.empty(1 << bits, np.float32)
    t = np.empty((1 << bits) - 1, np.float32)
    _check(load_library().rtq_lloyd_max(d, bits, c.ctypes.data, t.ctypes.data))
    return c, t


# ------------------------------------------------------------------ device objects

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RTQ_F32
    if t.dtype == torch.bfloat16:
        return RTQ_BF16
    if t.dtype == torch.int32:
        return RTQ_I32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_local_workspace(torch, nbytes: int, device, stream):
    """A temporary workspace for one call.  torch's caching allocator may hand its memory to other
    work once it is freed; recording the launch stream makes that wait for the call's kernels when
    they run on a stream other than the current one."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Rpbh:
    """A rotation descriptor on the device (perm int32[d], signs int8[d], h = 64)."""

    def __init__(self, perm, signs, h: int = 64):
        torch = _torch()
        self.perm = perm if isinstance(perm, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(perm))
        self.signs = signs if isinstance(signs, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(signs))
        self.d = int(self.perm.numel())
        self.h = h
        self._c = _Rpbh(self.d, h, _ptr(self.perm), _ptr(self.signs))

    @classmethod
    def from_seed(cls, seed: int, d: int, device="cuda"):
        perm, signs = rpbh_make(seed, d)
        torch = _torch()
        return cls(torch.from_numpy(perm).to(device), torch.from_numpy(signs).to(device))

    @classmethod
    def without_permutation(cls, seed: int, d: int, device="cuda"):
        """Block Hadamard with the seeded signs and no permutation (perm = identity): the ablation
        of the permutation step (OrbitQuant article, sections 2.3 and 3.3)."""
        _, signs = rpbh_make(seed, d)
        torch = _torch()
        return cls(torch.arange(d, dtype=torch.int32, device=device), torch.from_numpy(signs).to(device))

    @property
    def c(self):
        return ctypes.byref(self._c)


class Codebook:
    """A Lloyd-Max codebook on the device (centroids fp32[2^bits], boundaries fp32[2^bits - 1])."""

    def __init__(self, bits: int, centroids, boundaries):
        self.bits = bits
        self.centroids = centroids
        self.boundaries = boundaries
        self._c = _Codebook(bits, _ptr(centroids), _ptr(boundaries))

    @classmethod
    def for_dim(cls, d: int, bits: int, device="cuda"):
        c, t = lloyd_max(d, bits)
        torch = _torch()
        return cls(bits, torch.from_numpy(c).to(device), torch.from_numpy(t).to(device))

    @property
    def c(self):
        return ctypes.byref(self._c)


def _cb(cb):
    return None if cb is None else cb.c


# ------------------------------------------------------------------ device calls

def rpbh_rotate(x, y, R: Rpbh, inverse: bool = False, stream=None):
    """y = Pi x (or x = Pi^T y when inverse) row by row."""
    rows = x.shape[0] if x.dim() > 1 else 0
    _check(load_library().rtq_rpbh_rotate(_ptr(x), _dtype_code(x), _ptr(y), _dtype_code(y), rows, R.c,
                                          1 if inverse else 0, _stream(stream)))
    return y


def quantize_rows(x, codes, scale, R: Rpbh | None = None, mode: int = RTQ_INT8, cb: Codebook | None = None,
                  eps: float = 0.0, stream=None):
    """Rotate (if R) and quantise each row of x into codes + per-row scale/norm."""
    rows, d = x.shape
    need = tiled_code_bytes(rows, d, mode, cb.bits if cb is not None else 8)
    if codes.numel() * codes.element_size() < need:
        raise ValueError(f"tiled codes need {need} bytes (rows padded to a multiple of 256)")
    _check(load_library().rtq_quantize_rows(_ptr(x), _dtype_code(x), rows, d, None if R is None else R.c, mode,
                                            _cb(cb), ctypes.c_float(eps), _ptr(codes), _ptr(scale),
                                            _dtype_code(scale), _stream(stream)))
    return codes, scale


def qgemm(a_codes, a_scale, w_codes, w_scale, y, d: int, mode: int = RTQ_INT8, cb_a: Codebook | None = None,
          cb_w: Codebook | None = None, stream=None, workspace=None, n_tokens: int | None = None,
          n_out: int | None = None):
    """y = dequantised product of activation and weight codes (rotation already cancelled).
    With a workspace (qgemm_workspace() bytes) this is rtq_qgemm_ws: a partial last round of tiles
    is shared along d (stream-K runs after a full round, equal K ranges otherwise).
    T and N default to the codes' first dimensions; pass n_tokens / n_out for tiled codes (whose
    buffers hold rows padded to a multiple of 256), or take them from y."""
    T = a_codes.shape[0] if n_tokens is None else n_tokens
    N = w_codes.shape[0] if n_out is None else n_out
    lib = load_library()
    if workspace is None:
        _check(lib.rtq_qgemm(_ptr(a_codes), _ptr(a_scale), T, _ptr(w_codes), _ptr(w_scale), _dtype_code(w_scale), N,
                             d, mode, _cb(cb_a), _cb(cb_w), _ptr(y), _dtype_code(y), _stream(stream)))
    else:
        _check(lib.rtq_qgemm_ws(_ptr(a_codes), _ptr(a_scale), T, _ptr(w_codes), _ptr(w_scale), _dtype_code(w_scale),
                                N, d, mode, _cb(cb_a), _cb(cb_w), _ptr(y), _dtype_code(y), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def qgemm_workspace() -> int:
    """Bytes of workspace qgemm(..., workspace=...) uses on the current device."""
    return int(load_library().rtq_qgemm_workspace())


def new_qgemm_workspace(device="cuda"):
    """A zero-filled workspace for qgemm(..., workspace=...): its arrival counters must start at
    zero, and every product that completes leaves them zero again, so it can be reused as is."""
    return _torch().zeros(qgemm_workspace(), dtype=_torch().uint8, device=device)


def rotated_qlinear_workspace(T: int, d: int, mode: int = RTQ_INT8, bits_a: int = 8) -> int:
    return int(load_library().rtq_rotated_qlinear_workspace(T, d, mode, bits_a))


def rotated_qlinear(x, R: Rpbh, w_codes, w_scale, y, mode: int = RTQ_INT8, cb_a: Codebook | None = None,
                    cb_w: Codebook | None = None, workspace=None, stream=None):
    """The online layer: rotate + quantise x, then the quantised product, on one stream."""
    torch = _torch()
    T = x.shape[0]
    bits_a = cb_a.bits if (mode in _CODEBOOK_MODES and cb_a is not None) else 8
    N = y.shape[1]
    need = rotated_qlinear_workspace(T, R.d, mode, bits_a)
    if workspace is None:
        workspace = _stream_local_workspace(torch, max(need, 16), x.device, stream)
    _check(load_library().rtq_rotated_qlinear(_ptr(x), _dtype_code(x), T, R.c, _ptr(w_codes), _ptr(w_scale),
                                              _dtype_code(w_scale), N, mode, _cb(cb_a), _cb(cb_w),
                                              _ptr(y), _dtype_code(y), _ptr(workspace), workspace.numel(),
                                              _stream(stream)))
    return y


def rotated_qlinear_noalloc(x, R: Rpbh, w_codes, w_scale, y, mode: int = RTQ_INT8, cb_a: Codebook | None = None,
                            cb_w: Codebook | None = None, stream=None):
    """The online layer with no workspace: the activation codes and scales go to the library's
    static device scratch (NOALLOC_SCRATCH_BYTES per GPU; calls on one GPU must not overlap)."""
    T = x.shape[0]
    _check(load_library().rtq_rotated_qlinear_noalloc(_ptr(x), _dtype_code(x), T, R.c, _ptr(w_codes), _ptr(w_scale),
                                                      _dtype_code(w_scale), y.shape[1], mode, _cb(cb_a),
                                                      _cb(cb_w), _ptr(y), _dtype_code(y), _stream(stream)))
    return y


# ------------------------------------------------------------------ asymmetric INT8

def quantize_rows_asym(x, codes, scale, zero, code_sum, R: Rpbh, stream=None):
    """Rotate and quantise each row with a scale and a zero point (int8 codes, scale, int32 zero
    point, int32 code sum per row)."""
    rows, d = x.shape
    _check(load_library().rtq_quantize_rows_asym(_ptr(x), _dtype_code(x), rows, d, R.c, _ptr(codes), _ptr(scale),
                                                 _dtype_code(scale), _ptr(zero), _ptr(code_sum), _stream(stream)))
    return codes, scale, zero, code_sum


def qgemm_asym(a_codes, a_scale, a_zero, a_sum, w_codes, w_scale, w_zero, w_sum, y, d: int, stream=None,
               workspace=None):
    """y = a_scale * w_scale * sum_j (qa - za)(qw - zw)."""
    T, N = a_codes.shape[0], w_codes.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().rtq_qgemm_asym(_ptr(a_codes), _ptr(a_scale), _ptr(a_zero), _ptr(a_sum), T, _ptr(w_codes),
                                         _ptr(w_scale), _dtype_code(w_scale), _ptr(w_zero), _ptr(w_sum), N, d, _ptr(y),
                                         _dtype_code(y), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def rotated_qlinear_asym_workspace(T: int, d: int) -> int:
    return int(load_library().rtq_rotated_qlinear_asym_workspace(T, d))


def rotated_qlinear_asym(x, R: Rpbh, w_codes, w_scale, w_zero, w_sum, y, workspace=None, stream=None):
    """The online asymmetric layer: rotate + quantise x with zero points, then the zero-point product."""
    torch = _torch()
    T = x.shape[0]
    if workspace is None:
        workspace = _stream_local_workspace(torch, max(rotated_qlinear_asym_workspace(T, R.d), 16), x.device, stream)
    _check(load_library().rtq_rotated_qlinear_asym(_ptr(x), _dtype_code(x), T, R.c, _ptr(w_codes), _ptr(w_scale),
                                                   _dtype_code(w_scale), _ptr(w_zero), _ptr(w_sum), w_codes.shape[0],
                                                   _ptr(y), _dtype_code(y), _ptr(workspace), workspace.numel(),
                                                   _stream(stream)))
    return y
