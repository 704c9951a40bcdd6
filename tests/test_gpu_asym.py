"""GPU parity of asymmetric INT8 (a scale and a zero point per row, the scale-and-zero-point form
of INT8 the pages name: "INT8旋转量化是什么" section 3 and the int8 image-model page).

Tolerances: scales and zero points bit-exact; codes equal except one-step differences where the
oracle's fp32 v/s lies within 1e-6 relative of a rounding boundary; code sums consistent with the
codes; accumulators sum_j (qa - za)(qw - zw) bit-exact; y within 1e-5 relative (fp32 output of the
same codes) and the 2e-2 bound against the oracle's layer for bf16 I/O."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
from _helpers import bf16_host, dense_pi, int8_mismatches_allowed, rel_fro, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _quant_asym(xh, d, seed, scale_bf16):
    rows = xh.shape[0]
    codes = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.bfloat16 if scale_bf16 else torch.float32, device="cuda")
    zero = torch.empty(rows, dtype=torch.int32, device="cuda")
    csum = torch.empty(rows, dtype=torch.int32, device="cuda")
    rtq.quantize_rows_asym(to_dev(xh, "bf16"), codes, scale, zero, csum, rtq.Rpbh.from_seed(seed, d))
    torch.cuda.synchronize()
    s = workloads.bf16_bits_to_f32(bf16_host(scale)) if scale_bf16 else scale.cpu().numpy()
    return codes, scale, zero, csum, s


@pytest.mark.parametrize("d,rows,scale_bf16,dist", [(256, 130, False, "t3"), (4096, 71, True, "w"),
                                                    (4096, 200, False, "t3"), (16384, 5, True, "w"),
                                                    (1024, 40, False, "shift")])
def test_quantize_asym_matches_oracle(d, rows, scale_bf16, dist):
    xf = workloads.small_case(1700 + d + rows, rows, d, "t3" if dist == "shift" else dist)
    if dist == "shift":
        xf = xf + np.float32(3.0)       # rows far from zero mean: the rotated mean lands on a few coordinates
    xf[1] = 0.0                                                        # a zero row
    xh = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xh)
    seed = 29 + d
    codes, _, zero, csum, s = _quant_asym(xh, d, seed, scale_bf16)
    _, rot = oracle.rotate(xf, dense_pi(seed, d))
    qo, so, zo, sumo, pre = oracle.quantize_int8_asym(rot, scale_bf16)
    assert np.array_equal(s, so)
    assert np.array_equal(zero.cpu().numpy(), zo)
    q = codes.cpu().numpy()
    n_bad, n_out = int8_mismatches_allowed(q, qo, pre)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"
    got_sum = csum.cpu().numpy().astype(np.int64)
    assert np.array_equal(got_sum, q.astype(np.int64).sum(1))
    assert np.abs(got_sum - sumo).sum() <= n_bad
    assert s[1] == 0 and zero.cpu().numpy()[1] == 0 and not q[1].any()


@pytest.mark.parametrize("T,N,d", [(130, 200, 256), (257, 129, 128), (64, 384, 4096), (300, 700, 2048),
                                   (33, 70, 16384)])
def test_qgemm_asym_accumulators_bit_exact(T, N, d):
    rng = np.random.default_rng(T + N + d)
    qa = rng.integers(-128, 128, size=(T, d)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(N, d)).astype(np.int8)
    za = rng.integers(-128, 128, size=T).astype(np.int32)
    zw = rng.integers(-128, 128, size=N).astype(np.int32)
    sa = qa.astype(np.int64).sum(1).astype(np.int32)
    sw = qw.astype(np.int64).sum(1).astype(np.int32)
    ref = oracle.gemm_int8_asym(qa, za, qw, zw)
    ones_t, ones_n = to_dev(np.ones(T, np.float32)), to_dev(np.ones(N, np.float32))
    ws = rtq.new_qgemm_workspace()
    for workspace in (None, ws):
        acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
        rtq.qgemm_asym(to_dev(qa), ones_t, to_dev(za), to_dev(sa), to_dev(qw), ones_n, to_dev(zw), to_dev(sw), acc, d,
                       workspace=workspace)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref)
    # scaled outputs: the same accumulators times a_scale * w_scale
    s_a = (rng.random(T) * 0.1 + 0.01).astype(np.float32)
    r_wb = oracle.to_bf16_bits(rng.random(N) * 0.1 + 0.01)
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    rtq.qgemm_asym(to_dev(qa), to_dev(s_a), to_dev(za), to_dev(sa), to_dev(qw), to_dev(r_wb, "bf16"), to_dev(zw),
                   to_dev(sw), y, d, workspace=ws)
    torch.cuda.synchronize()
    want = oracle.rescale_int8(ref, s_a, oracle.bf16_bits_to_f32(r_wb))
    assert rel_fro(y.cpu().numpy().astype(np.float64), want) <= 1e-5


def test_qgemm_asym_stream_k_sampled():
    # 288 tiles at d = 1024: stream-K runs of 18 stages cross tile edges, and the zero-point terms
    # are applied once, after the two partial sums are added
    T, N, d = 4608, 4096, 1024
    rng = np.random.default_rng(41)
    qa = rng.integers(-128, 128, size=(T, d)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(N, d)).astype(np.int8)
    za = rng.integers(-128, 128, size=T).astype(np.int32)
    zw = rng.integers(-128, 128, size=N).astype(np.int32)
    sa = qa.astype(np.int64).sum(1).astype(np.int32)
    sw = qw.astype(np.int64).sum(1).astype(np.int32)
    rows = np.concatenate([np.sort(rng.choice(T, 40, replace=False)), [0, T - 1]])
    ref = oracle.gemm_int8_asym(qa[rows], za[rows], qw, zw)
    ws = rtq.new_qgemm_workspace()
    acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
    ones_t, ones_n = to_dev(np.ones(T, np.float32)), to_dev(np.ones(N, np.float32))
    rtq.qgemm_asym(to_dev(qa), ones_t, to_dev(za), to_dev(sa), to_dev(qw), ones_n, to_dev(zw), to_dev(sw), acc, d,
                   workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), ref)


@pytest.mark.parametrize("yt", ["f32", "bf16"])
def test_qgemm_asym_stream_k_equals_whole(yt):
    # 289 tiles with ragged edges and N % 8 != 0: the stream-K product (partials added before
    # the zero-point terms and the scales) equals the product launched whole, bit for bit
    T, N, d = 4100, 4100, 1024
    rng = np.random.default_rng(43)
    qa = rng.integers(-128, 128, size=(T, d)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(N, d)).astype(np.int8)
    za = rng.integers(-128, 128, size=T).astype(np.int32)
    zw = rng.integers(-128, 128, size=N).astype(np.int32)
    sa = qa.astype(np.int64).sum(1).astype(np.int32)
    sw = qw.astype(np.int64).sum(1).astype(np.int32)
    s_a = to_dev((rng.random(T) * 0.1 + 0.01).astype(np.float32))
    r_w = to_dev(oracle.to_bf16_bits(rng.random(N) * 0.1 + 0.01), "bf16")
    dt = torch.float32 if yt == "f32" else torch.bfloat16
    args = (to_dev(qa), s_a, to_dev(za), to_dev(sa), to_dev(qw), r_w, to_dev(zw), to_dev(sw))
    y0 = torch.empty((T, N), dtype=dt, device="cuda")
    y1 = torch.empty((T, N), dtype=dt, device="cuda")
    rtq.qgemm_asym(*args, y0, d)
    ws = rtq.new_qgemm_workspace()
    rtq.qgemm_asym(*args, y1, d, workspace=ws)
    torch.cuda.synchronize()
    iv = torch.int32 if yt == "f32" else torch.int16
    assert torch.equal(y0.view(iv), y1.view(iv))


@pytest.mark.parametrize("T,N,d", [(200, 256, 4096), (70, 130, 256), (33, 96, 16384)])
def test_asym_layer_small(T, N, d):
    xf = workloads.small_case(1800 + d, T, d, "t3")
    wf = workloads.small_case(1801 + d, N, d, "w")
    xh, wh = workloads.f32_to_bf16_bits(xf), workloads.f32_to_bf16_bits(wf)
    xf, wf = workloads.bf16_bits_to_f32(xh), workloads.bf16_bits_to_f32(wh)
    seed = 57
    R = rtq.Rpbh.from_seed(seed, d)
    wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
    ws_ = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    wz = torch.empty(N, dtype=torch.int32, device="cuda")
    wsum = torch.empty(N, dtype=torch.int32, device="cuda")
    rtq.quantize_rows_asym(to_dev(wh, "bf16"), wq, ws_, wz, wsum, R)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rtq.rotated_qlinear_asym(to_dev(xh, "bf16"), R, wq, ws_, wz, wsum, y)
    torch.cuda.synchronize()
    pi = dense_pi(seed, d)
    wo = oracle.weights_int8_asym(wf, pi, True)
    assert int8_mismatches_allowed(wq.cpu().numpy(), wo["q"], wo["pre"])[1] == 0
    assert np.array_equal(wz.cpu().numpy(), wo["zero"])
    out = oracle.qlinear_int8_asym(xf, pi, wo)
    got = workloads.bf16_bits_to_f32(bf16_host(y))
    assert rel_fro(got, out["y"]) <= 2e-2
    # the same codes give the same accumulators: the layer's error is the bf16 output rounding
    assert rel_fro(got, out["y"]) <= 4e-3


def test_asym_dit_shape_sampled():
    # the W8A8 DiT layer (4608 x 4096 -> 16384) with zero points, launched whole
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh, wh = workloads.dit_activations_bf16(d), workloads.dit_weight_bf16("mlp_up")
    T = xh.shape[0]
    seed = workloads.RPBH_SEED[d]
    R = rtq.Rpbh.from_seed(seed, d)
    wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
    ws_ = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    wz = torch.empty(N, dtype=torch.int32, device="cuda")
    wsum = torch.empty(N, dtype=torch.int32, device="cuda")
    rtq.quantize_rows_asym(_bf16(wh), wq, ws_, wz, wsum, R)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rtq.rotated_qlinear_asym(_bf16(xh), R, wq, ws_, wz, wsum, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = np.concatenate([[T - 1], np.sort(rng.choice(np.arange(0, T - 1), 5, replace=False))])
    cols = np.concatenate([[N - 1], np.sort(rng.choice(np.arange(0, N - 1), 40, replace=False))])
    pi = dense_pi(seed, d)
    wo = oracle.weights_int8_asym(workloads.bf16_bits_to_f32(wh[cols]), pi, True)
    assert int8_mismatches_allowed(wq.cpu().numpy()[cols], wo["q"], wo["pre"])[1] == 0
    out = oracle.qlinear_int8_asym(workloads.bf16_bits_to_f32(xh[rows]), pi, wo)
    got = workloads.bf16_bits_to_f32(bf16_host(y))[np.ix_(rows, cols)]
    assert rel_fro(got, out["y"]) <= 4e-3


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
