"""Shared helpers for the GPU parity tests (marshalling and comparison only)."""
import functools
import math

import numpy as np

import oracle


def to_dev(a, dtype=None):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_host(t):
    """bf16 device tensor -> uint16 bit patterns on the host."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=4)
def dense_pi(seed: int, d: int):
    perm, signs = oracle.rpbh_descriptor(seed, d)
    return oracle.rpbh_dense(d, 64, perm, signs)


def int8_mismatches_allowed(q_gpu, q_orc, pre_orc):
    """Allowance for INT8 codes: equal, or one step apart where the oracle's fp32
    pre-rounding value lies within 1e-6 relative of the rounding boundary k + 1/2."""
    diff = q_gpu.astype(np.int32) - q_orc.astype(np.int32)
    bad = diff != 0
    if not bad.any():
        return 0, 0
    t = pre_orc[bad].astype(np.float64)
    half = np.floor(t) + 0.5
    near = np.abs(t - half) <= 1e-6 * np.maximum(np.abs(half), 1.0)
    ok = (np.abs(diff[bad]) == 1) & near
    return int(bad.sum()), int((~ok).sum())


def codebook_mismatches_allowed(c_gpu, c_orc, u_orc, bounds, d):
    """Codes equal, or one cell apart where the oracle's u lies within 1e-6 * max(|t_k|, 1/sqrt(d))
    of the boundary t_k between them."""
    diff = c_gpu.astype(np.int32) - c_orc.astype(np.int32)
    bad = diff != 0
    if not bad.any():
        return 0, 0
    u = u_orc[bad].astype(np.float64)
    tb = bounds.astype(np.float64)
    k = np.argmin(np.abs(u[:, None] - tb[None, :]), axis=1)
    tol = 1e-6 * np.maximum(np.abs(tb[k]), 1.0 / math.sqrt(d))
    ok = (np.abs(diff[bad]) == 1) & (np.abs(u - tb[k]) <= tol)
    return int(bad.sum()), int((~ok).sum())


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def int8_table(centroids):
    """(S, v) with S = fl32(127 / max|c|) and v_k = rint(fl32(c_k * S)) as int8 (the int8 codebook
    rule of include/rtq.h, computed with numpy fp32 arithmetic, independently of the library)."""
    c = np.asarray(centroids, np.float32)
    s = np.float32(127.0) / np.max(np.abs(c))
    v = np.rint(c * s).astype(np.int8)
    return s, v


def codes_of(values, table):
    """Invert the (injective) table: int8 values -> codes."""
    lookup = {int(v): k for k, v in enumerate(table)}
    assert len(lookup) == len(table)
    flat = np.array([lookup.get(int(v), -1) for v in values.ravel()], np.int64)
    assert (flat >= 0).all(), "value outside the codebook table"
    return flat.reshape(values.shape)


def tile_codes(codes):
    """Row-major int8 codes [rows][d] -> the tiled layout of RTQ_INT8_TILED (a flat int8 array of
    ceil(rows/256)*256*d bytes; padding rows are zero): block (row // 256, j // 64) of 16 KB holds
    [256 rows][64 bytes], chunk c of a row's 64 bytes at chunk c ^ ((row >> 2) & 3)."""
    codes = np.asarray(codes, np.int8)
    rows, d = codes.shape
    rp = -(-rows // 256) * 256
    full = np.zeros((rp, d), np.int8)
    full[:rows] = codes
    # [tile][256][slice][4 chunks][16] -> [tile][slice][256][4 chunks (swizzled)][16]
    v = full.reshape(rp // 256, 256, d // 64, 4, 16)
    r = np.arange(256)
    perm = (np.arange(4)[None, :] ^ ((r[:, None] >> 2) & 3))           # [256][4]: chunk c -> slot
    out = np.empty((rp // 256, d // 64, 256, 4, 16), np.int8)
    for c in range(4):
        out[:, :, r, perm[:, c], :] = v[:, :, :, c, :].transpose(0, 2, 1, 3)
    return out.reshape(-1)


def untile_codes(buf, rows, d):
    """Inverse of tile_codes: the first `rows` rows as a row-major [rows][d] int8 array."""
    buf = np.asarray(buf).view(np.int8).reshape(-1)
    rp = -(-rows // 256) * 256
    v = buf[:rp * d].reshape(rp // 256, d // 64, 256, 4, 16)
    r = np.arange(256)
    perm = (np.arange(4)[None, :] ^ ((r[:, None] >> 2) & 3))
    full = np.empty((rp // 256, 256, d // 64, 4, 16), np.int8)
    for c in range(4):
        full[:, :, :, c, :] = v[:, :, r, perm[:, c], :].transpose(0, 2, 1, 3)
    return full.reshape(rp, d)[:rows]


def tile_packed(codes, bits):
    """Row-major packed codebook codes [rows][d * bits / 8] (uint8) -> the tiled code layout of
    RTQ_CODEBOOK_TILED (a flat uint8 array of ceil(rows/256)*256*d*bits/8 bytes; padding rows are
    zero): block (row // 256, j // 64) holds [256 rows][8 * bits bytes], a row's bytes being its
    packed codes of elements 64 * (j // 64) .. +64 unchanged."""
    codes = np.asarray(codes, np.uint8)
    rows, wrow = codes.shape
    rb = 8 * bits
    assert wrow % rb == 0
    rp = -(-rows // 256) * 256
    full = np.zeros((rp, wrow), np.uint8)
    full[:rows] = codes
    # [tile][256][slice][rb] -> [tile][slice][256][rb]
    return full.reshape(rp // 256, 256, wrow // rb, rb).transpose(0, 2, 1, 3).reshape(-1).copy()


def untile_packed(buf, rows, d, bits):
    """Inverse of tile_packed: the first `rows` rows as row-major [rows][d * bits / 8] uint8."""
    buf = np.asarray(buf).view(np.uint8).reshape(-1)
    rb = 8 * bits
    rp = -(-rows // 256) * 256
    v = buf[:rp * d * bits // 8].reshape(rp // 256, d // 64, 256, rb)
    return v.transpose(0, 2, 1, 3).reshape(rp, d * bits // 8)[:rows]
