"""Seeded synthetic inputs for the rotated low-bit linear layer.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic (no rotation, no scale, no code, no
codebook), so both the CPU oracle and the GPU path can take their inputs from
it.  Every array comes from ``numpy.random.default_rng(seed)`` (PCG64), is
drawn in fp32, and is rounded to bf16 (nearest-even) where the workload
stores bf16.

The shapes follow the DiT the pages describe: a 7B-parameter, 32-layer,
single-stream image DiT ("INT8旋转量化是什么？图像生成模型轻量化全解", section 2)
with hidden size 4096 and MLP width 16384, 4096 latent-patch tokens plus 512
text tokens.  Heavy-tailed activations with a few outlier channels and
weights with a few outlier input columns stand in for the outliers the pages
say break plain quantisation (same page, section 2; OrbitQuant article,
section 1).  No public benchmark, dataset or model weights are used.
"""
from __future__ import annotations

import functools
from dataclasses import dataclass

import numpy as np

H_BLOCK = 64  # Walsh-Hadamard block size used throughout


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns, nearest-even (inputs are finite)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _outlier_columns(seed, d: int, frac_or_count) -> np.ndarray:
    rng = np.random.default_rng(seed)
    count = frac_or_count if isinstance(frac_or_count, int) else int(round(frac_or_count * d))
    return np.sort(rng.choice(d, size=count, replace=False))


def gaussian_weight(seed, outlier_seed, n_out: int, d_in: int, std: float, outlier_frac_or_count,
                    outlier_gain: float) -> np.ndarray:
    """W[n_out][d_in] ~ N(0, std^2) in fp32 with some input columns scaled by outlier_gain."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n_out, d_in), dtype=np.float32)
    w *= np.float32(std)
    cols = _outlier_columns(outlier_seed, d_in, outlier_frac_or_count)
    w[:, cols] *= np.float32(outlier_gain)
    return w


def student_t_activations(seed, outlier_seed, tokens: int, d: int, nu: float, outlier_frac_or_count,
                          outlier_gain: float) -> np.ndarray:
    """x[tokens][d] ~ Student-t(nu) in fp32 with some channels scaled by outlier_gain."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(nu, size=(tokens, d)).astype(np.float32)
    cols = _outlier_columns(outlier_seed, d, outlier_frac_or_count)
    x[:, cols] *= np.float32(outlier_gain)
    return x


def gaussian_activations(seed, outlier_seed, tokens: int, d: int, outlier_count: int, outlier_gain: float):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, d), dtype=np.float32)
    cols = _outlier_columns(outlier_seed, d, outlier_count)
    x[:, cols] *= np.float32(outlier_gain)
    return x


# --------------------------------------------------------------------------
# The workloads.  Seeds for workload k: weights 1000k+1, activations 1000k+2,
# rotation descriptor 1000k+3, outlier picks 1000k+4.

DIT_TOKENS = 4096 + 512   # latent patches + text tokens
DIT_HIDDEN = 4096
DIT_MLP = 16384

# The rotation descriptor is one per input dimension and shared by every
# layer of that width (weights offline, activations online).
RPBH_SEED = {256: 1003, 4096: 2003, 16384: 2013}

# One DiT block's four linears as (name, d_out, d_in).
DIT_LINEARS = (
    ("qkv", 3 * DIT_HIDDEN, DIT_HIDDEN),
    ("attn_out", DIT_HIDDEN, DIT_HIDDEN),
    ("mlp_up", DIT_MLP, DIT_HIDDEN),
    ("mlp_down", DIT_HIDDEN, DIT_MLP),
)


@dataclass(frozen=True)
class Linear:
    name: str
    tokens: int
    d_in: int
    d_out: int
    io: str          # "f32" or "bf16"
    wbits: int       # 8 = symmetric INT8, 2/4 = Lloyd-Max codebook
    abits: int


TINY = Linear("tiny_w8a8_256x512_t128_f32", 128, 256, 512, "f32", 8, 8)
W8A8_DIT = Linear("w8a8_dit_mlp_up_4608x4096x16384_bf16", DIT_TOKENS, DIT_HIDDEN, DIT_MLP, "bf16", 8, 8)
W4A4_DIT = Linear("w4a4_dit_attn_out_4608x4096x4096_bf16", DIT_TOKENS, DIT_HIDDEN, DIT_HIDDEN, "bf16", 4, 4)
W2A4_DIT = Linear("w2a4_dit_mlp_down_4608x16384x4096_bf16", DIT_TOKENS, DIT_MLP, DIT_HIDDEN, "bf16", 2, 4)


@functools.lru_cache(maxsize=None)
def tiny_inputs():
    """d_in=256, d_out=512, 128 tokens, fp32.  W ~ N(0, 1/256) with 4 input
    columns x20; x ~ N(0,1) with 2 channels x30."""
    w = gaussian_weight(1001, 1004, 512, 256, 1.0 / 16.0, 4, 20.0)
    x = gaussian_activations(1002, [1004, 1], 128, 256, 2, 30.0)
    return {"w": w, "x": x, "rpbh_seed": RPBH_SEED[256]}


@functools.lru_cache(maxsize=None)
def dit_weight_bf16(name: str) -> np.ndarray:
    """One of the DiT block's linears, bf16 bits [d_out][d_in]:
    N(0, 0.02^2) plus 0.5% of the input columns scaled x15."""
    idx = [n for n, _, _ in DIT_LINEARS].index(name)
    _, d_out, d_in = DIT_LINEARS[idx]
    w = gaussian_weight([2001, idx], [2004, idx], d_out, d_in, 0.02, 0.005, 15.0)
    return f32_to_bf16_bits(w)


@functools.lru_cache(maxsize=None)
def dit_activations_bf16(d: int, tokens: int = DIT_TOKENS) -> np.ndarray:
    """bf16 bits [tokens][d]: Student-t(3) with 1% of the channels scaled x50."""
    seed = 3002 if d == DIT_HIDDEN else 5002
    oseed = 3004 if d == DIT_HIDDEN else 5004
    x = student_t_activations(seed, oseed, tokens, d, 3.0, 0.01, 50.0)
    return f32_to_bf16_bits(x)


@functools.lru_cache(maxsize=None)
def w4a4_weight_bf16() -> np.ndarray:
    """The attention-output shape (4096 x 4096) with the DiT weight statistics."""
    w = gaussian_weight(4001, 4004, DIT_HIDDEN, DIT_HIDDEN, 0.02, 0.005, 15.0)
    return f32_to_bf16_bits(w)


@functools.lru_cache(maxsize=None)
def w2a4_weight_bf16() -> np.ndarray:
    """The MLP-down shape (4096 x 16384) with the DiT weight statistics."""
    w = gaussian_weight(5001, [5004, 1], DIT_HIDDEN, DIT_MLP, 0.02, 0.005, 15.0)
    return f32_to_bf16_bits(w)


def small_case(seed: int, rows: int, d: int, dist: str = "t3", outlier_frac=0.01, gain=50.0) -> np.ndarray:
    """Small fp32 test matrices with the same value distributions, for parity at sizes the oracle
    finishes in seconds."""
    if dist == "t3":
        return student_t_activations(seed, [seed, 7], rows, d, 3.0, outlier_frac, gain)
    if dist == "w":
        return gaussian_weight(seed, [seed, 7], rows, d, 0.02, 0.005, 15.0)
    if dist == "normal":
        return gaussian_activations(seed, [seed, 7], rows, d, max(1, int(round(outlier_frac * d))), gain)
    raise ValueError(dist)


# --------------------------------------------------------------------------
# Inputs for the transform ablation (block Hadamard without the permutation, dense rotation).

def dit_activation_outlier_channels(d: int) -> np.ndarray:
    """The channels dit_activations_bf16(d) scales by x50 (sorted)."""
    oseed = 3004 if d == DIT_HIDDEN else 5004
    return _outlier_columns(oseed, d, 0.01)


def clustered_order(d: int, first: np.ndarray) -> np.ndarray:
    """A column order that puts the channels `first` at the front (so they fill the first
    ceil(len/64) blocks of 64) and keeps the rest in place order.  Applying it to the columns of
    both x and W leaves W x unchanged."""
    first = np.asarray(first, np.int64)
    rest = np.setdiff1d(np.arange(d, dtype=np.int64), first)
    return np.concatenate([first, rest])


@functools.lru_cache(maxsize=None)
def haar_orthogonal(seed: int, d: int) -> np.ndarray:
    """A Haar-distributed random orthogonal matrix [d][d] (fp32): the Q factor of a seeded
    Gaussian matrix, with the signs fixed by R's diagonal so the distribution is uniform."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q *= np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)
