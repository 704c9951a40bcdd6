"""GPU parity of the codebook path on the INT8 matrix cores (RTQ_CODEBOOK_I8).

The mode keeps the Lloyd-Max codes of the method and changes only the numbers the product sees:
each codebook enters as v_k = rint(c_k * S), S = 127 / max_k |c_k| (fp32 arithmetic, as the
header states).  So the tests check two things separately:
  * the integer part is exact: activation values are the table entries of the oracle's codes
    (same boundary allowance as the packed codes), the raw int32 accumulators equal the int64
    product of the tables bit for bit, and the bf16 output is that product rescaled by
    a_scale * w_scale / (S_a S_w) to within one bf16 ulp per element;
  * the whole layer stays within the layer's bound (2e-2 relative Frobenius, bf16 output) of
    the oracle's exact-centroid product.
The table is computed here from the oracle's centroids with numpy fp32 arithmetic (the rule in
include/rtq.h), independently of the library."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
import _dit_cases as dit_cases
from _dit_cases import bf16_within_one_ulp
from _helpers import bf16_host, codebook_mismatches_allowed, codes_of, dense_pi, int8_table, rel_fro, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def test_int8_tables_are_injective_and_symmetric():
    for d, bits in [(4096, 4), (16384, 4), (16384, 2), (256, 2), (1024, 4)]:
        s, v = int8_table(oracle.lloyd_max(bits, d)["centroids"])
        assert len(set(v.tolist())) == len(v)
        assert np.array_equal(v, -v[::-1])
        assert np.max(np.abs(v)) == 127


@pytest.mark.parametrize("d,rows,bits", [(4096, 130, 4), (16384, 6, 4), (256, 65, 2), (1024, 40, 4)])
def test_quantize_codebook_i8_values(d, rows, bits):
    xf = workloads.small_case(900 + d + bits, rows, d, "t3")
    xf[rows - 1] = 0.0
    xh = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xh)
    seed = 21 + d
    cb = rtq.Codebook.for_dim(d, bits)
    ref_cb = oracle.lloyd_max(bits, d)
    _, table = int8_table(ref_cb["centroids"])
    vals = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), vals, scale, rtq.Rpbh.from_seed(seed, d), rtq.RTQ_CODEBOOK_I8, cb, 1e-8)
    torch.cuda.synchronize()
    _, rot = oracle.rotate(xf, dense_pi(seed, d))
    co, so, u = oracle.quantize_codebook(rot, ref_cb["boundaries"], False, 1e-8)
    assert np.array_equal(scale.cpu().numpy(), so)
    got = codes_of(vals.cpu().numpy(), table)
    n_bad, n_out = codebook_mismatches_allowed(got, co, u, ref_cb["boundaries"], d)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"
    assert np.all(got[rows - 1] == (1 << bits) // 2 - 1)


def test_quantize_codebook_i8_fp32_input_without_rotation():
    # the generic row kernel (fp32 input, rows already rotated)
    d, rows, bits = 512, 33, 4
    rng = np.random.default_rng(5)
    xf = (rng.standard_normal((rows, d)) / np.sqrt(d)).astype(np.float32)
    cb = rtq.Codebook.for_dim(d, bits)
    ref_cb = oracle.lloyd_max(bits, d)
    _, table = int8_table(ref_cb["centroids"])
    vals = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xf), vals, scale, None, rtq.RTQ_CODEBOOK_I8, cb, 1e-8)
    torch.cuda.synchronize()
    co, so, u = oracle.quantize_codebook(xf, ref_cb["boundaries"], False, 1e-8)
    assert np.array_equal(scale.cpu().numpy(), so)
    got = codes_of(vals.cpu().numpy(), table)
    assert codebook_mismatches_allowed(got, co, u, ref_cb["boundaries"], d)[1] == 0


@pytest.mark.parametrize("bits_w", [4, 2])
@pytest.mark.parametrize("wst", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,d", [(130, 200, 256), (300, 521, 1024), (64, 384, 4096), (7, 9, 64), (257, 130, 128)])
def test_codebook_i8_gemm(bits_w, wst, T, N, d):
    rng = np.random.default_rng(T + 7 * N + d + bits_w)
    qa = rng.integers(0, 16, size=(T, d)).astype(np.uint8)
    qw = rng.integers(0, 1 << bits_w, size=(N, d)).astype(np.uint8)
    ocb_a, ocb_w = oracle.lloyd_max(4, d), oracle.lloyd_max(bits_w, d)
    sa_i, ta = int8_table(ocb_a["centroids"])
    sw_i, tw = int8_table(ocb_w["centroids"])
    s_a = (rng.random(T) * 10 + 1).astype(np.float32)
    if wst == "bf16":
        r_wb = oracle.to_bf16_bits(rng.random(N) + 0.5)
        r_w = oracle.bf16_bits_to_f32(r_wb)
        w_scale = to_dev(r_wb, "bf16")
    else:
        r_w = (rng.random(N) + 0.5).astype(np.float32)
        w_scale = to_dev(r_w)
    a_dev, w_dev = to_dev(ta[qa]), to_dev(oracle.pack(qw, bits_w))
    cba, cbw = rtq.Codebook.for_dim(d, 4), rtq.Codebook.for_dim(d, bits_w)
    # raw accumulators: the exact int64 product of the two int8 tables, bit for bit
    acc = ta[qa].astype(np.int64) @ tw[qw].astype(np.int64).T
    acc_gpu = torch.empty((T, N), dtype=torch.int32, device="cuda")
    rtq.qgemm(a_dev, to_dev(s_a), w_dev, w_scale, acc_gpu, d, rtq.RTQ_CODEBOOK_I8, cba, cbw)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rtq.qgemm(a_dev, to_dev(s_a), w_dev, w_scale, y, d, rtq.RTQ_CODEBOOK_I8, cba, cbw)
    torch.cuda.synchronize()
    assert np.array_equal(acc_gpu.cpu().numpy().astype(np.int64), acc)
    got = oracle.bf16_bits_to_f32(bf16_host(y))
    # rescaled: the same exact sums times s_t r_n / (S_a S_w), at most one bf16 ulp apart
    y_int = acc * s_a.astype(np.float64)[:, None] * r_w.astype(np.float64)[None, :] / (float(sa_i) * float(sw_i))
    assert np.all(bf16_within_one_ulp(got, y_int))
    # against the oracle's exact-centroid product: inside the bf16 bound
    ref = oracle.gemm_codebook(qa, qw, ocb_a["centroids"], ocb_w["centroids"], s_a, r_w)
    assert rel_fro(got, ref) <= 2e-2


@pytest.mark.parametrize("bits_w,T,N,d", [(4, 200, 256, 4096), (2, 70, 130, 16384), (4, 33, 65, 256),
                                          (2, 300, 520, 1024)])
def test_codebook_i8_layer_small(bits_w, T, N, d):
    xf = workloads.small_case(710 + d, T, d, "t3")
    wf = workloads.small_case(711 + d, N, d, "w")
    xh, wh = workloads.f32_to_bf16_bits(xf), workloads.f32_to_bf16_bits(wf)
    xf, wf = workloads.bf16_bits_to_f32(xh), workloads.bf16_bits_to_f32(wh)
    seed = 47
    R = rtq.Rpbh.from_seed(seed, d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, 4), rtq.Codebook.for_dim(d, bits_w)
    wcodes = torch.empty((N, d * bits_w // 8), dtype=torch.uint8, device="cuda")
    wnorm = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wcodes, wnorm, R, rtq.RTQ_CODEBOOK, cb_w, 0.0)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    need = rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_CODEBOOK_I8, 4)
    split = (rtq.qgemm_workspace() + 255) // 256 * 256      # the product's K-split region
    assert need == ((T * d + 255) // 256) * 256 + ((4 * T + 255) // 256) * 256 + split
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wcodes, wnorm, y, rtq.RTQ_CODEBOOK_I8, cb_a, cb_w, workspace=ws)
    torch.cuda.synchronize()
    pi = dense_pi(seed, d)
    ocb_a, ocb_w = oracle.lloyd_max(4, d), oracle.lloyd_max(bits_w, d)
    wo = oracle.weights_codebook(wf, pi, ocb_w, bits_w)
    assert codebook_mismatches_allowed(oracle.unpack(wcodes.cpu().numpy(), d, bits_w), wo["codes"], wo["u"],
                                       ocb_w["boundaries"], d)[1] == 0
    out = oracle.qlinear_codebook(xf, pi, wo, ocb_a, ocb_w, 4)
    # the workspace holds the activations' int8 codebook values and their norms
    _, ta = int8_table(ocb_a["centroids"])
    a_codes = codes_of(ws[:T * d].view(T, d).cpu().numpy().view(np.int8), ta)
    assert codebook_mismatches_allowed(a_codes, out["act"]["codes"], out["act"]["u"], ocb_a["boundaries"], d)[1] == 0
    off = ((T * d + 255) // 256) * 256
    assert np.array_equal(ws[off:off + 4 * T].view(torch.float32).cpu().numpy(), out["act"]["norm"])
    got = workloads.bf16_bits_to_f32(bf16_host(y))
    assert rel_fro(got, out["y"]) <= 2e-2


@pytest.mark.parametrize("variant", ["w4a4", "w2a4"])
def test_codebook_i8_dit_shape_sampled(variant):
    # the benchmark's codebook layers (4-bit activations as int8 codebook values on the INT8
    # matrix cores), launched on the full tensors as the benchmark does; 64 tokens x 256 channels
    # covering every output tile (all tiles are shared along d by stream-K runs at these shapes)
    ref = dit_cases.codebook_sample(variant)
    d, N, bits_w, bits_a = ref["d"], ref["N"], ref["bits_w"], ref["bits_a"]
    _, _, _, _, wgen = dit_cases.CODEBOOK_VARIANTS[variant]
    xh, wh = workloads.dit_activations_bf16(d), wgen()
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, bits_a), rtq.Codebook.for_dim(d, bits_w)
    wcodes = torch.empty((N, d * bits_w // 8), dtype=torch.uint8, device="cuda")
    wnorm = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wcodes, wnorm, R, rtq.RTQ_CODEBOOK, cb_w, 0.0)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_CODEBOOK_I8, bits_a), dtype=torch.uint8,
                       device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wcodes, wnorm, y, rtq.RTQ_CODEBOOK_I8, cb_a, cb_w, workspace=work)
    torch.cuda.synchronize()
    rows, cols, wo, ao = ref["rows"], ref["cols"], ref["wo"], ref["ao"]
    ocb_a, ocb_w = ref["ocb_a"], ref["ocb_w"]
    w_codes = oracle.unpack(wcodes.cpu().numpy()[cols], d, bits_w)
    assert codebook_mismatches_allowed(w_codes, wo["codes"], wo["u"], ocb_w["boundaries"], d)[1] == 0
    assert np.array_equal(workloads.bf16_bits_to_f32(bf16_host(wnorm))[cols], wo["norm"])
    a_codes = codes_of(work[:T * d].view(T, d).cpu().numpy().view(np.int8)[rows], ref["ta"])
    assert codebook_mismatches_allowed(a_codes, ao["codes"], ao["u"], ocb_a["boundaries"], d)[1] == 0
    off = ((T * d + 255) // 256) * 256
    assert np.array_equal(work[off:off + 4 * T].view(torch.float32).cpu().numpy()[rows], ao["norm"])
    got = workloads.bf16_bits_to_f32(bf16_host(y))[np.ix_(rows, cols)]
    # against the oracle's exact-centroid product: the bf16 bound
    assert rel_fro(got, ref["y"]) <= 2e-2
    # element by element against the same codes through the int8 tables (exact int64 sums):
    # where a token's and a channel's codes equal the oracle's, at most one bf16 ulp apart
    same = np.all(a_codes == ao["codes"], axis=1)[:, None] & np.all(w_codes == wo["codes"], axis=1)[None, :]
    assert same.mean() > 0.9
    assert np.all(dit_cases.bf16_within_one_ulp(got, ref["y_int8"])[same])
