"""GPU parity of the fused RPBH rotate/quantise kernel against the CPU oracle.

Tolerances (stated per test): rotated rows bit-exact on bf16 and small-integer inputs and within
1e-5 relative L2 per row otherwise; INT8 and packed codebook codes bit-exact except one-step
differences where the oracle's fp32 value lies within 1e-6 relative of the rounding/codebook
boundary; scales and norms bit-exact."""
import math

import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
from _helpers import (bf16_host, codebook_mismatches_allowed, dense_pi, int8_mismatches_allowed, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _rpbh(seed, d):
    return rtq.Rpbh.from_seed(seed, d)


def _case(seed, rows, d, dist="t3"):
    return workloads.small_case(seed, rows, d, dist)


@pytest.mark.parametrize("d,rows", [(64, 5), (256, 130), (1024, 33), (4096, 19), (16384, 3)])
def test_rotate_fp32_matches_dense_product(d, rows):
    x = _case(100 + d, rows, d, "normal")
    R = _rpbh(7 + d, d)
    y = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    rtq.rpbh_rotate(to_dev(x), y, R)
    torch.cuda.synchronize()
    _, ref = oracle.rotate(x, dense_pi(7 + d, d))
    got = y.cpu().numpy()
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() <= 1e-5
    # fp64 butterflies are exact here in all but pathological cases: expect identical bits
    assert np.mean(got == ref) > 0.9999


@pytest.mark.parametrize("d", [256, 4096])
def test_rotate_integer_inputs_bit_exact(d):
    rng = np.random.default_rng(5)
    x = rng.integers(-1000, 1001, size=(9, d)).astype(np.float32)
    R = _rpbh(3, d)
    y = torch.empty((9, d), dtype=torch.float32, device="cuda")
    rtq.rpbh_rotate(to_dev(x), y, R)
    _, ref = oracle.rotate(x, dense_pi(3, d))
    assert np.array_equal(y.cpu().numpy(), ref)


@pytest.mark.parametrize("d,rows", [(256, 67), (4096, 21), (16384, 2)])
def test_rotate_bf16_inputs_bit_exact_and_bf16_output(d, rows):
    xb = workloads.f32_to_bf16_bits(_case(200 + d, rows, d))
    x = workloads.bf16_bits_to_f32(xb)
    R = _rpbh(11, d)
    y32 = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    y16 = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    xd = to_dev(xb, "bf16")
    rtq.rpbh_rotate(xd, y32, R)
    rtq.rpbh_rotate(xd, y16, R)
    _, ref = oracle.rotate(x, dense_pi(11, d))
    # bf16 inputs: every partial sum is exact, so the once-rounded result is identical
    assert np.array_equal(y32.cpu().numpy(), ref)
    assert np.array_equal(bf16_host(y16), oracle.to_bf16_bits(ref.astype(np.float64)))


@pytest.mark.parametrize("d", [64, 4096, 16384])
def test_inverse_undoes_rotation_on_device(d):
    # Pi^T Pi = I (OrbitQuant article, 2.2): rotating and rotating back returns the input.
    rows = 6
    x = _case(300 + d, rows, d)
    R = _rpbh(13, d)
    xd = to_dev(x)
    y = torch.empty_like(xd)
    back = torch.empty_like(xd)
    rtq.rpbh_rotate(xd, y, R)
    rtq.rpbh_rotate(y, back, R, inverse=True)
    got = back.cpu().numpy()
    assert np.max(np.abs(got - x)) <= 2e-6 * np.max(np.abs(x))
    # and the inverse itself matches the oracle's Pi^T product
    _, ref = oracle.rotate(y.cpu().numpy(), dense_pi(13, d), inverse=True)
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() <= 1e-6


def _quant_int8(xh, xt, d, seed, scale_bf16, rotate=True):
    rows = xh.shape[0]
    R = _rpbh(seed, d) if rotate else None
    x = to_dev(xh, "bf16") if xt == "bf16" else to_dev(xh)
    codes = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.bfloat16 if scale_bf16 else torch.float32, device="cuda")
    rtq.quantize_rows(x, codes, scale, R, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    s = bf16_host(scale) if scale_bf16 else scale.cpu().numpy()
    if scale_bf16:
        s = workloads.bf16_bits_to_f32(s)
    return codes.cpu().numpy(), s


@pytest.mark.parametrize("d,rows,xt,scale_bf16", [
    (256, 130, "f32", False),      # tiny fp32 layer shape, ragged row count
    (4096, 71, "bf16", True),      # DiT weights: bf16 row scales
    (4096, 300, "bf16", False),    # DiT tokens: fp32 token scales
    (16384, 5, "bf16", True),
    (64, 257, "f32", False),
])
def test_quantize_int8_matches_oracle(d, rows, xt, scale_bf16):
    xf = _case(400 + d + rows, rows, d, "w" if scale_bf16 else "t3")
    xf[min(3, rows - 1)] = 0.0                                    # a zero row
    if xt == "bf16":
        xh = workloads.f32_to_bf16_bits(xf)
        xf = workloads.bf16_bits_to_f32(xh)
    else:
        xh = xf
    seed = 17 + d
    q, s = _quant_int8(xh, xt, d, seed, scale_bf16)
    _, rot = oracle.rotate(xf, dense_pi(seed, d))
    qo, so, pre = oracle.quantize_int8(rot, scale_bf16)
    assert np.array_equal(s, so)
    n_bad, n_out = int8_mismatches_allowed(q, qo, pre)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"
    assert s[min(3, rows - 1)] == 0 and not q[min(3, rows - 1)].any()


def test_quantize_int8_prerotated_rows():
    d, rows = 1024, 40
    xf = _case(31, rows, d)
    q, s = _quant_int8(xf, "f32", d, 0, False, rotate=False)
    qo, so, pre = oracle.quantize_int8(xf, False)
    assert np.array_equal(s, so)
    assert int8_mismatches_allowed(q, qo, pre)[1] == 0


@pytest.mark.parametrize("d,rows,bits,weight", [
    (4096, 130, 4, False),   # W4A4 activations: fp32 token norms, eps = 1e-8
    (4096, 37, 4, True),     # W4A4 weights: bf16 row norms, eps = 0
    (16384, 6, 4, False),    # W2A4 activations at d = 16384
    (16384, 9, 2, True),     # W2A4 weights
    (256, 65, 2, False),
    # several rows per wave with an all-zero weight row (norm 0, eps = 0) among nonzero ones: the
    # boundary-grid table of every row in the wave is built by lanes of all its rows
    (1024, 23, 4, True),
    (512, 21, 3, True),
])
def test_quantize_codebook_matches_oracle(d, rows, bits, weight):
    xf = _case(500 + d + bits, rows, d, "w" if weight else "t3")
    xf[rows - 1] = 0.0
    xh = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xh)
    seed = 19 + d
    cb = rtq.Codebook.for_dim(d, bits)
    ref_cb = oracle.lloyd_max(bits, d)
    assert np.array_equal(cb.boundaries.cpu().numpy(), ref_cb["boundaries"])
    eps = 0.0 if weight else 1e-8
    codes = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device="cuda")
    scale = torch.empty(rows, dtype=torch.bfloat16 if weight else torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), codes, scale, _rpbh(seed, d), rtq.RTQ_CODEBOOK, cb, eps)
    torch.cuda.synchronize()
    s = workloads.bf16_bits_to_f32(bf16_host(scale)) if weight else scale.cpu().numpy()
    _, rot = oracle.rotate(xf, dense_pi(seed, d))
    co, so, u = oracle.quantize_codebook(rot, ref_cb["boundaries"], weight, eps if not weight else 1e-8)
    assert np.array_equal(s, so)
    got = oracle.unpack(codes.cpu().numpy(), d, bits)
    n_bad, n_out = codebook_mismatches_allowed(got, co, u, ref_cb["boundaries"], d)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"
    # zero row: u = 0 -> lower cell of the middle boundary
    assert np.all(got[rows - 1] == (1 << bits) // 2 - 1)


def test_quantize_is_deterministic():
    d, rows = 4096, 200
    xh = workloads.f32_to_bf16_bits(_case(77, rows, d))
    x = to_dev(xh, "bf16")
    R = _rpbh(5, d)
    cb = rtq.Codebook.for_dim(d, 4)
    outs = []
    for _ in range(2):
        c = torch.empty((rows, d // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty(rows, dtype=torch.float32, device="cuda")
        rtq.quantize_rows(x, c, s, R, rtq.RTQ_CODEBOOK, cb, 1e-8)
        outs.append((c.cpu().numpy(), s.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
