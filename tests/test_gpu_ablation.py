"""GPU parity of the transform ablation (OrbitQuant article, sections 2.3 and 3.3): block Hadamard
without the permutation (perm = identity, the seeded signs) through the same kernels, and a dense
rotation applied as a library GEMM before the pre-rotated quantiser.

Tolerances: codes bit-exact except one-step differences where the oracle's fp32 value lies within
1e-6 relative of the rounding/codebook boundary; scales and norms bit-exact; the dense rotation
within 1e-5 relative L2 per row (an fp32 GEMM against the oracle's fp64 product)."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
from _helpers import bf16_host, codebook_mismatches_allowed, int8_mismatches_allowed, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _bh_pi(seed, d):
    _, signs = oracle.rpbh_descriptor(seed, d)
    return oracle.rpbh_dense(d, 64, np.arange(d, dtype=np.int32), signs)


@pytest.mark.parametrize("d,rows,scale_bf16", [(256, 130, False), (4096, 37, False), (4096, 19, True),
                                               (16384, 3, True)])
def test_block_hadamard_int8_matches_oracle(d, rows, scale_bf16):
    seed = 40 + d
    xf = workloads.small_case(seed, rows, d, "w" if scale_bf16 else "t3")
    xh = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xh)
    R = rtq.Rpbh.without_permutation(seed, d)
    assert np.array_equal(R.perm.cpu().numpy(), np.arange(d))
    codes = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.bfloat16 if scale_bf16 else torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), codes, scale, R, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    s = workloads.bf16_bits_to_f32(bf16_host(scale)) if scale_bf16 else scale.cpu().numpy()
    _, rot = oracle.rotate(xf, _bh_pi(seed, d))
    qo, so, pre = oracle.quantize_int8(rot, scale_bf16)
    assert np.array_equal(s, so)
    n_bad, n_out = int8_mismatches_allowed(codes.cpu().numpy(), qo, pre)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"


def test_block_hadamard_codebook_matches_oracle():
    d, rows, bits = 4096, 24, 4
    seed = 77
    xh = workloads.f32_to_bf16_bits(workloads.small_case(seed, rows, d))
    xf = workloads.bf16_bits_to_f32(xh)
    R = rtq.Rpbh.without_permutation(seed, d)
    cb = rtq.Codebook.for_dim(d, bits)
    codes = torch.empty((rows, d // 2), dtype=torch.uint8, device="cuda")
    norm = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), codes, norm, R, rtq.RTQ_CODEBOOK, cb, 1e-8)
    torch.cuda.synchronize()
    ocb = oracle.lloyd_max(bits, d)
    _, rot = oracle.rotate(xf, _bh_pi(seed, d))
    co, no, uo = oracle.quantize_codebook(rot, ocb["boundaries"], False, 1e-8)
    assert np.array_equal(norm.cpu().numpy(), no)
    got = oracle.unpack(codes.cpu().numpy(), d, bits)
    n_bad, n_out = codebook_mismatches_allowed(got, co, uo, ocb["boundaries"], d)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"


def test_dense_rotation_then_prerotated_quantise_matches_oracle():
    d, rows = 1024, 33
    x = workloads.small_case(91, rows, d)
    q = workloads.haar_orthogonal(91, d)
    xd = to_dev(x)
    rot = xd @ to_dev(q).t()                     # the dense rotation as an fp32 library GEMM
    torch.cuda.synchronize()
    _, ref = oracle.rotate(x, q.astype(np.float64))
    got = rot.cpu().numpy()
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() <= 1e-5
    codes = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(rot, codes, scale, None, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    qo, so, pre = oracle.quantize_int8(got, False)
    assert np.array_equal(scale.cpu().numpy(), so)
    n_bad, n_out = int8_mismatches_allowed(codes.cpu().numpy(), qo, pre)
    assert n_out == 0
