"""CPU oracle for the rotated low-bit linear layer -- TEST INFRASTRUCTURE.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.  The arithmetic lives in ``oracle.c`` (plain C: dense
rotation matrix, double accumulation, IEEE fp32 division, round-half-even,
counting codebook search, triple-loop GEMM); this module only marshals numpy
arrays into it and strings the steps together in the order the pages give.

Pages cited (by title and section):
  [OQ]  OrbitQuant article (hotelren.com/news/3376620), sections 2.1-2.3, 4.2.
  [CR2] "量化旋转主模型是什么？一文读懂低比特图像生成模型", section 4 (q = round(RW/s)).

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against closed forms, invariants, textbook or
library special cases, or brute force on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
I64P = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
I8P = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
U16P = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
U64P = np.ctypeslib.ndpointer(dtype=np.uint64, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
               "-D_GNU_SOURCE", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    c_i64, c_i32, c_int, c_u64, c_f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_uint64, ctypes.c_float
    lib.orc_splitmix64_stream.argtypes = [c_u64, c_i64, U64P]
    lib.orc_splitmix64_stream.restype = None
    lib.orc_rpbh_descriptor.argtypes = [c_u64, c_i32, I32P, I8P]
    lib.orc_rpbh_descriptor.restype = c_int
    lib.orc_rpbh_dense.argtypes = [c_i32, c_i32, I32P, I8P, F64P]
    lib.orc_rpbh_dense.restype = c_int
    lib.orc_rotate_rows.argtypes = [F64P, c_i32, F32P, c_i64, c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.orc_rotate_rows.restype = None
    lib.orc_to_bf16.argtypes = [F64P, c_i64, U16P]
    lib.orc_to_bf16.restype = None
    lib.orc_quant_int8_rows.argtypes = [F32P, c_i64, c_i32, c_int, I8P, F32P, ctypes.c_void_p]
    lib.orc_quant_int8_rows.restype = None
    lib.orc_quant_int8_asym_rows.argtypes = [F32P, c_i64, c_i32, c_int, I8P, F32P, I32P, I64P, ctypes.c_void_p]
    lib.orc_quant_int8_asym_rows.restype = None
    lib.orc_gemm_int8_asym.argtypes = [I8P, I32P, I8P, I32P, c_i64, c_i64, c_i32, I64P]
    lib.orc_gemm_int8_asym.restype = None
    lib.orc_quant_codebook_rows.argtypes = [F32P, c_i64, c_i32, c_int, c_f32, c_i32, F32P, U8P, F32P,
                                            ctypes.c_void_p]
    lib.orc_quant_codebook_rows.restype = None
    lib.orc_pack.argtypes = [U8P, c_i64, c_i32, c_i32, U8P]
    lib.orc_pack.restype = c_int
    lib.orc_unpack.argtypes = [U8P, c_i64, c_i32, c_i32, U8P]
    lib.orc_unpack.restype = c_int
    lib.orc_lloyd_max.argtypes = [c_i32, c_i32, F64P, F64P, F32P, F32P]
    lib.orc_lloyd_max.restype = c_int
    lib.orc_gemm_int8.argtypes = [I8P, I8P, c_i64, c_i64, c_i32, I64P]
    lib.orc_gemm_int8.restype = None
    lib.orc_rescale_int8.argtypes = [I64P, F32P, F32P, c_i64, c_i64, F64P]
    lib.orc_rescale_int8.restype = None
    lib.orc_gemm_codebook.argtypes = [U8P, U8P, F32P, F32P, F32P, F32P, c_i64, c_i64, c_i32, F64P]
    lib.orc_gemm_codebook.restype = None
    lib.orc_matmul_f64.argtypes = [F32P, F32P, c_i64, c_i64, c_i32, F64P]
    lib.orc_matmul_f64.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = c_int
    _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


# --------------------------------------------------------------------------
# RPBH rotation ([OQ] section 2.3)

def splitmix64(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().orc_splitmix64_stream(ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), n, out)
    return out


def rpbh_descriptor(seed: int, d: int):
    """Seeded permutation (gather form) and Rademacher signs of length d."""
    perm = np.empty(d, np.int32)
    signs = np.empty(d, np.int8)
    if _load().orc_rpbh_descriptor(ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), d, perm, signs) != 0:
        raise ValueError("bad d")
    return perm, signs


def rpbh_dense(d: int, h: int, perm: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """The explicit d x d matrix Pi_d = blkdiag(H_h D_i) P_pi (fp64)."""
    pi = np.empty((d, d), np.float64)
    if _load().orc_rpbh_dense(d, h, _c(perm, np.int32), _c(signs, np.int8), pi) != 0:
        raise ValueError("d must be a positive multiple of h")
    return pi


def rotate(x: np.ndarray, pi: np.ndarray, inverse: bool = False):
    """Rows of x (fp32) times Pi (or Pi^T): returns (fp64 exact-order sums, fp32 once-rounded)."""
    x = _c(x, np.float32)
    rows, d = x.shape
    out64 = np.empty((rows, d), np.float64)
    out32 = np.empty((rows, d), np.float32)
    _load().orc_rotate_rows(_c(pi, np.float64), d, x, rows, 1 if inverse else 0,
                            out64.ctypes.data, out32.ctypes.data)
    return out64, out32


# --------------------------------------------------------------------------
# number formats

def to_bf16_bits(x) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of float64 (or float32) values."""
    x = np.asarray(x, np.float64)
    flat = _c(x.reshape(-1), np.float64)
    out = np.empty(flat.shape, np.uint16)
    _load().orc_to_bf16(flat, flat.size, out)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# quantisation

def quantize_int8(v: np.ndarray, scale_bf16: bool):
    """Symmetric per-row INT8. Returns (q int8, stored scale as fp32, pre-rounding v/s)."""
    v = _c(v, np.float32)
    rows, d = v.shape
    q = np.empty((rows, d), np.int8)
    s = np.empty(rows, np.float32)
    pre = np.empty((rows, d), np.float32)
    _load().orc_quant_int8_rows(v, rows, d, 1 if scale_bf16 else 0, q, s, pre.ctypes.data)
    return q, s, pre


def quantize_int8_asym(v: np.ndarray, scale_bf16: bool):
    """Asymmetric per-row INT8 (scale + zero point, range widened to contain 0).
    Returns (q int8, stored scale fp32, zero point int32, code sum int64, pre-rounding v/s)."""
    v = _c(v, np.float32)
    rows, d = v.shape
    q = np.empty((rows, d), np.int8)
    s = np.empty(rows, np.float32)
    z = np.empty(rows, np.int32)
    csum = np.empty(rows, np.int64)
    pre = np.empty((rows, d), np.float32)
    _load().orc_quant_int8_asym_rows(v, rows, d, 1 if scale_bf16 else 0, q, s, z, csum, pre.ctypes.data)
    return q, s, z, csum, pre


def gemm_int8_asym(qa: np.ndarray, za: np.ndarray, qw: np.ndarray, zw: np.ndarray) -> np.ndarray:
    qa, qw = _c(qa, np.int8), _c(qw, np.int8)
    T, d = qa.shape
    N = qw.shape[0]
    acc = np.empty((T, N), np.int64)
    _load().orc_gemm_int8_asym(qa, _c(za, np.int32), qw, _c(zw, np.int32), T, N, d, acc)
    return acc


def quantize_codebook(v: np.ndarray, bounds: np.ndarray, is_weight: bool, eps: float = 1e-8):
    """Row-norm + Lloyd-Max direction codes. Returns (codes uint8 unpacked, stored norm fp32, u)."""
    v = _c(v, np.float32)
    rows, d = v.shape
    bounds = _c(bounds, np.float32)
    codes = np.empty((rows, d), np.uint8)
    nrm = np.empty(rows, np.float32)
    u = np.empty((rows, d), np.float32)
    _load().orc_quant_codebook_rows(v, rows, d, 1 if is_weight else 0, ctypes.c_float(eps), bounds.size, bounds,
                                    codes, nrm, u.ctypes.data)
    return codes, nrm, u


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    rows, d = codes.shape
    out = np.empty((rows, d * bits // 8), np.uint8)
    if _load().orc_pack(codes, rows, d, bits, out) != 0:
        raise ValueError("bits must be 2, 3, 4, 6 or 8 with d * bits a multiple of 8")
    return out


def unpack(packed: np.ndarray, d: int, bits: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    rows = packed.shape[0]
    out = np.empty((rows, d), np.uint8)
    if _load().orc_unpack(packed, rows, d, bits, out) != 0:
        raise ValueError("bits must be 2, 3, 4, 6 or 8 with d * bits a multiple of 8")
    return out


def lloyd_max(bits: int, d: int) -> dict:
    """Lloyd-Max codebook for N(0, 1/d) ([OQ] section 4.2)."""
    L = 1 << bits
    cu = np.empty(L, np.float64)
    tu = np.empty(L - 1, np.float64)
    c32 = np.empty(L, np.float32)
    t32 = np.empty(L - 1, np.float32)
    it = _load().orc_lloyd_max(bits, d, cu, tu, c32, t32)
    if it < 0:
        raise ValueError("bits must be in 1..8")
    return {"c_unit": cu, "t_unit": tu, "centroids": c32, "boundaries": t32, "iters": it}


# --------------------------------------------------------------------------
# products

def gemm_int8(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    qa = _c(qa, np.int8)
    qw = _c(qw, np.int8)
    T, d = qa.shape
    N = qw.shape[0]
    acc = np.empty((T, N), np.int64)
    _load().orc_gemm_int8(qa, qw, T, N, d, acc)
    return acc


def rescale_int8(acc: np.ndarray, a_scale: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    acc = _c(acc, np.int64)
    T, N = acc.shape
    y = np.empty((T, N), np.float64)
    _load().orc_rescale_int8(acc, _c(a_scale, np.float32), _c(w_scale, np.float32), T, N, y)
    return y


def gemm_codebook(qa, qw, ca, cw, s_a, r_w) -> np.ndarray:
    qa = _c(qa, np.uint8)
    qw = _c(qw, np.uint8)
    T, d = qa.shape
    N = qw.shape[0]
    y = np.empty((T, N), np.float64)
    _load().orc_gemm_codebook(qa, qw, _c(ca, np.float32), _c(cw, np.float32), _c(s_a, np.float32),
                              _c(r_w, np.float32), T, N, d, y)
    return y


def matmul_f64(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    T, d = x.shape
    N = w.shape[0]
    y = np.empty((T, N), np.float64)
    _load().orc_matmul_f64(x, w, T, N, d, y)
    return y


# --------------------------------------------------------------------------
# the layer, step by step ([OQ] sections 2.1 and 2.2)

def weights_int8(w: np.ndarray, pi: np.ndarray, scale_bf16: bool):
    """Offline: W' = W Pi^T (row n is Pi w_n), per-row symmetric INT8."""
    _, w_rot = rotate(w, pi)
    q, s, pre = quantize_int8(w_rot, scale_bf16)
    return {"rot": w_rot, "q": q, "scale": s, "pre": pre}


def activations_int8(x: np.ndarray, pi: np.ndarray):
    """Online: x' = Pi x, per-token symmetric INT8 with an fp32 scale."""
    _, x_rot = rotate(x, pi)
    q, s, pre = quantize_int8(x_rot, False)
    return {"rot": x_rot, "q": q, "scale": s, "pre": pre}


def weights_codebook(w: np.ndarray, pi: np.ndarray, cb: dict, bits: int):
    """Offline: W' = W Pi^T, bf16 row norm r', direction codes Q_b(w'/r'), packed."""
    _, w_rot = rotate(w, pi)
    codes, r, u = quantize_codebook(w_rot, cb["boundaries"], True)
    return {"rot": w_rot, "codes": codes, "packed": pack(codes, bits), "norm": r, "u": u}


def activations_codebook(x: np.ndarray, pi: np.ndarray, cb: dict, bits: int, eps: float = 1e-8):
    """Online: x' = Pi x, s = ||x'||, codes Q_b(x'/(s+eps)), packed."""
    _, x_rot = rotate(x, pi)
    codes, s, u = quantize_codebook(x_rot, cb["boundaries"], False, eps)
    return {"rot": x_rot, "codes": codes, "packed": pack(codes, bits), "norm": s, "u": u}


def qlinear_int8(x: np.ndarray, pi: np.ndarray, wq: dict) -> dict:
    a = activations_int8(x, pi)
    acc = gemm_int8(a["q"], wq["q"])
    y = rescale_int8(acc, a["scale"], wq["scale"])
    return {"act": a, "acc": acc, "y": y}


def weights_int8_asym(w: np.ndarray, pi: np.ndarray, scale_bf16: bool):
    """Offline: W' = W Pi^T, per-row asymmetric INT8."""
    _, w_rot = rotate(w, pi)
    q, s, z, csum, pre = quantize_int8_asym(w_rot, scale_bf16)
    return {"rot": w_rot, "q": q, "scale": s, "zero": z, "sum": csum, "pre": pre}


def qlinear_int8_asym(x: np.ndarray, pi: np.ndarray, wq: dict) -> dict:
    """Online: x' = Pi x, per-token asymmetric INT8 (fp32 scale), the zero-point product, rescale."""
    _, x_rot = rotate(x, pi)
    q, s, z, csum, pre = quantize_int8_asym(x_rot, False)
    a = {"rot": x_rot, "q": q, "scale": s, "zero": z, "sum": csum, "pre": pre}
    acc = gemm_int8_asym(q, z, wq["q"], wq["zero"])
    y = rescale_int8(acc, s, wq["scale"])
    return {"act": a, "acc": acc, "y": y}


def qlinear_codebook(x: np.ndarray, pi: np.ndarray, wq: dict, cb_a: dict, cb_w: dict, bits_a: int) -> dict:
    a = activations_codebook(x, pi, cb_a, bits_a)
    y = gemm_codebook(a["codes"], wq["codes"], cb_a["centroids"], cb_w["centroids"], a["norm"], wq["norm"])
    return {"act": a, "y": y}
