"""Sampled oracle results at the DiT shapes, for the full-shape GPU parity tests.

The GPU launches the whole layer; the oracle computes only the sampled tokens and output
channels (dense rotation of those rows, then quantisation and the product).  The samples cover
every 256 x 256 output tile: each tile's first and last row and column, plus seeded random
indices, so the last (ragged) tiles and the tiles shared along d by stream-K runs are all met.
Results are cached per process, since several tests compare against the same samples."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import workloads
from _helpers import dense_pi, int8_table

TILE = 256


def tile_sample(n: int, count: int, seed: int, tile: int = TILE) -> np.ndarray:
    """`count` sorted distinct indices in [0, n): the first and last index of every tile of `tile`
    indices, then seeded random ones."""
    edges = set()
    for t0 in range(0, n, tile):
        edges.add(t0)
        edges.add(min(n, t0 + tile) - 1)
    assert len(edges) <= count, (n, count)
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(n), np.fromiter(edges, np.int64))
    extra = rng.choice(rest, count - len(edges), replace=False)
    return np.sort(np.concatenate([np.fromiter(edges, np.int64), extra]))


def bf16_within_one_ulp(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per element: is `got` (bf16 values as fp32) at most one bf16 ulp from the bf16 rounding of
    `ref` (fp64)?  Two roundings of nearly the same value differ by at most one ulp."""
    refb = oracle.bf16_bits_to_f32(oracle.to_bf16_bits(ref))
    ulp = np.spacing(np.abs(refb).astype(np.float32)).astype(np.float64) * 65536.0
    return np.abs(got.astype(np.float64) - refb.astype(np.float64)) <= ulp


@functools.lru_cache(maxsize=None)
def w8a8_sample():
    """W8A8 DiT MLP-up (4608 x 4096 -> 16384): 64 tokens x 256 channels through the oracle."""
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh = workloads.dit_activations_bf16(d)
    wh = workloads.dit_weight_bf16("mlp_up")
    T = xh.shape[0]
    rows = tile_sample(T, 64, 99)
    cols = tile_sample(N, 256, 100)
    pi = dense_pi(workloads.RPBH_SEED[d], d)
    wo = oracle.weights_int8(workloads.bf16_bits_to_f32(wh[cols]), pi, True)
    ao = oracle.activations_int8(workloads.bf16_bits_to_f32(xh[rows]), pi)
    acc = oracle.gemm_int8(ao["q"], wo["q"])
    y = oracle.rescale_int8(acc, ao["scale"], wo["scale"])
    return {"rows": rows, "cols": cols, "wo": wo, "ao": ao, "acc": acc, "y": y}


CODEBOOK_VARIANTS = {
    # name: (d, N, bits_w, bits_a, weight generator)
    "w4a4": (workloads.DIT_HIDDEN, workloads.DIT_HIDDEN, 4, 4, workloads.w4a4_weight_bf16),
    "w2a4": (workloads.DIT_MLP, workloads.DIT_HIDDEN, 2, 4, workloads.w2a4_weight_bf16),
    "w3a3": (workloads.DIT_HIDDEN, workloads.DIT_HIDDEN, 3, 3, workloads.w4a4_weight_bf16),
    "w4a6": (workloads.DIT_HIDDEN, workloads.DIT_HIDDEN, 4, 6, workloads.w4a4_weight_bf16),
}


@functools.lru_cache(maxsize=None)
def codebook_sample(variant: str):
    """A codebook DiT layer: 64 tokens x 256 channels through the oracle (codes, norms, the exact
    codebook product) and the product of the same codes through the int8 codebook tables (the
    RTQ_CODEBOOK_I8 rule, computed here with numpy from the oracle's centroids)."""
    d, N, bits_w, bits_a, wgen = CODEBOOK_VARIANTS[variant]
    xh = workloads.dit_activations_bf16(d)
    wh = wgen()
    T = xh.shape[0]
    rows = tile_sample(T, 64, 97)
    cols = tile_sample(N, 256, 96)
    pi = dense_pi(workloads.RPBH_SEED[d], d)
    ocb_a, ocb_w = oracle.lloyd_max(bits_a, d), oracle.lloyd_max(bits_w, d)
    wo = oracle.weights_codebook(workloads.bf16_bits_to_f32(wh[cols]), pi, ocb_w, bits_w)
    ao = oracle.activations_codebook(workloads.bf16_bits_to_f32(xh[rows]), pi, ocb_a, bits_a)
    y = oracle.gemm_codebook(ao["codes"], wo["codes"], ocb_a["centroids"], ocb_w["centroids"], ao["norm"],
                             wo["norm"])
    sa, ta = int8_table(ocb_a["centroids"])
    sw, tw = int8_table(ocb_w["centroids"])
    acc8 = ta[ao["codes"]].astype(np.int64) @ tw[wo["codes"]].astype(np.int64).T
    y8 = acc8 * ao["norm"].astype(np.float64)[:, None] * wo["norm"].astype(np.float64)[None, :] / (
        float(sa) * float(sw))
    return {"rows": rows, "cols": cols, "wo": wo, "ao": ao, "y": y, "y_int8": y8, "ta": ta,
            "ocb_a": ocb_a, "ocb_w": ocb_w, "d": d, "N": N, "bits_w": bits_w, "bits_a": bits_a}
