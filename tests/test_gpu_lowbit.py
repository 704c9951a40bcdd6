"""GPU parity of the W3A3 and W4A6 variants (OrbitQuant article, sections 3.2-3.3): 3-bit weight codes
(packed as one LSB-first bit stream, 8 codes per 3 bytes), 3- and 6-bit activation codes written as
their int8 codebook values, and the product on the INT8 matrix cores.

Tolerances as for the other codebook modes: codes equal except one-cell differences where the
oracle's u lies within 1e-6 * max(|t_k|, 1/sqrt(d)) of the boundary between them; norms bit-exact;
the product's integer part against an int64 reference of the int8 tables (1e-5 fp32 output, 4e-3
bf16), and the layer against the oracle's exact-centroid product at the 2e-2 bf16 bound."""
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


def test_int8_tables_of_three_and_six_bit_codebooks_are_injective():
    # the int8 rounding keeps 8 and 64 levels distinct (the six-bit levels are >= 2 apart)
    for d in (256, 1024, 4096, 16384):
        for bits in (3, 6):
            _, v = int8_table(oracle.lloyd_max(bits, d)["centroids"])
            assert len(set(v.tolist())) == len(v)
            assert np.array_equal(v, -v[::-1])
            assert np.min(np.diff(v.astype(np.int32))) >= (2 if bits == 6 else 10)


@pytest.mark.parametrize("d,rows,weight", [(256, 70, True), (1024, 33, False), (4096, 45, True), (4096, 64, False),
                                           (16384, 4, True)])
def test_quantize_three_bit_packed_codes(d, rows, weight):
    bits = 3
    xf = workloads.small_case(1300 + d + rows, rows, d, "w" if weight else "t3")
    xf[rows // 2] = 0.0
    xh = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xh)
    seed = 61 + d
    cb = rtq.Codebook.for_dim(d, bits)
    ocb = oracle.lloyd_max(bits, d)
    codes = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device="cuda")
    norm = torch.empty(rows, dtype=torch.bfloat16 if weight else torch.float32, device="cuda")
    eps = 0.0 if weight else 1e-8
    rtq.quantize_rows(to_dev(xh, "bf16"), codes, norm, rtq.Rpbh.from_seed(seed, d), rtq.RTQ_CODEBOOK, cb, eps)
    torch.cuda.synchronize()
    _, rot = oracle.rotate(xf, dense_pi(seed, d))
    co, no, uo = oracle.quantize_codebook(rot, ocb["boundaries"], weight, eps)
    got_norm = workloads.bf16_bits_to_f32(bf16_host(norm)) if weight else norm.cpu().numpy()
    assert np.array_equal(got_norm, no)
    # the bytes are the oracle's packing of the GPU's codes, and the codes are the oracle's
    got = oracle.unpack(codes.cpu().numpy(), d, bits)
    assert np.array_equal(oracle.pack(got, bits), codes.cpu().numpy())
    n_bad, n_out = codebook_mismatches_allowed(got, co, uo, ocb["boundaries"], d)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("d,rows", [(256, 65), (1024, 20), (4096, 70), (16384, 5)])
def test_quantize_int8_codebook_values(bits, d, rows):
    xf = workloads.small_case(1400 + d + bits, rows, d, "t3")
    xf[rows - 1] = 0.0
    xh = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xh)
    seed = 23 + d
    cb = rtq.Codebook.for_dim(d, bits)
    ocb = oracle.lloyd_max(bits, d)
    _, table = int8_table(ocb["centroids"])
    vals = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    norm = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), vals, norm, rtq.Rpbh.from_seed(seed, d), rtq.RTQ_CODEBOOK_I8, cb, 1e-8)
    torch.cuda.synchronize()
    _, rot = oracle.rotate(xf, dense_pi(seed, d))
    co, no, uo = oracle.quantize_codebook(rot, ocb["boundaries"], False, 1e-8)
    assert np.array_equal(norm.cpu().numpy(), no)
    got = codes_of(vals.cpu().numpy(), table)
    n_bad, n_out = codebook_mismatches_allowed(got, co, uo, ocb["boundaries"], d)
    assert n_out == 0, f"{n_bad} mismatches, {n_out} outside the boundary allowance"
    assert np.all(got[rows - 1] == (1 << bits) // 2 - 1)   # zero row: u = 0 sits on the middle boundary


@pytest.mark.parametrize("bits_w,bits_a", [(3, 3), (4, 6), (3, 6), (2, 3)])
@pytest.mark.parametrize("T,N,d", [(130, 200, 256), (300, 521, 1024), (64, 384, 4096), (257, 130, 128)])
def test_lowbit_gemm_integer_part_and_bound(bits_w, bits_a, T, N, d):
    rng = np.random.default_rng(T + 3 * N + d + 10 * bits_w + bits_a)
    qa = rng.integers(0, 1 << bits_a, size=(T, d)).astype(np.uint8)
    qw = rng.integers(0, 1 << bits_w, size=(N, d)).astype(np.uint8)
    ocb_a, ocb_w = oracle.lloyd_max(bits_a, d), oracle.lloyd_max(bits_w, d)
    sa_i, ta = int8_table(ocb_a["centroids"])
    sw_i, tw = int8_table(ocb_w["centroids"])
    s_a = (rng.random(T) * 10 + 1).astype(np.float32)
    r_wb = oracle.to_bf16_bits(rng.random(N) + 0.5)
    r_w = oracle.bf16_bits_to_f32(r_wb)
    acc = ta[qa].astype(np.int64) @ tw[qw].astype(np.int64).T
    for yt in ("i32", "bf16"):
        y = torch.empty((T, N), dtype=torch.int32 if yt == "i32" else torch.bfloat16, device="cuda")
        rtq.qgemm(to_dev(ta[qa]), to_dev(s_a), to_dev(oracle.pack(qw, bits_w)), to_dev(r_wb, "bf16"), y, d,
                  rtq.RTQ_CODEBOOK_I8, rtq.Codebook.for_dim(d, bits_a), rtq.Codebook.for_dim(d, bits_w))
        torch.cuda.synchronize()
        if yt == "i32":   # raw accumulators: the int64 product of the tables, bit for bit
            assert np.array_equal(y.cpu().numpy().astype(np.int64), acc)
            continue
        got = oracle.bf16_bits_to_f32(bf16_host(y))
        y_int = acc * s_a.astype(np.float64)[:, None] * r_w.astype(np.float64)[None, :] / (float(sa_i) * float(sw_i))
        assert np.all(bf16_within_one_ulp(got, y_int))
        ref = oracle.gemm_codebook(qa, qw, ocb_a["centroids"], ocb_w["centroids"], s_a, r_w)
        assert rel_fro(got, ref) <= 2e-2


def test_three_bit_weights_with_k_split_bit_exact_integer_part():
    # 288 tiles of 256 x 256 with d = 8192: the tiles are shared along d by stream-K runs; the
    # decode of 24-byte rows at each range's start must match the unsplit product exactly (same
    # int32 sums)
    T, N, d = 4608, 4096, 8192
    rng = np.random.default_rng(5)
    qa = rng.integers(0, 8, size=(T, d)).astype(np.uint8)
    qw = rng.integers(0, 8, size=(N, d)).astype(np.uint8)
    cb = rtq.Codebook.for_dim(d, 3)
    _, ta = int8_table(oracle.lloyd_max(3, d)["centroids"])
    a = to_dev(ta[qa])
    w = to_dev(oracle.pack(qw, 3))
    s_a = to_dev(np.ones(T, np.float32))
    s_w = to_dev(np.ones(N, np.float32))
    y0 = torch.empty((T, N), dtype=torch.int32, device="cuda")
    y1 = torch.empty((T, N), dtype=torch.int32, device="cuda")
    rtq.qgemm(a, s_a, w, s_w, y0, d, rtq.RTQ_CODEBOOK_I8, cb, cb)
    ws = rtq.new_qgemm_workspace()
    rtq.qgemm(a, s_a, w, s_w, y1, d, rtq.RTQ_CODEBOOK_I8, cb, cb, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    rows = np.array([0, 1000, 4607])
    acc = ta[qa[rows]].astype(np.int64) @ ta[qw].astype(np.int64).T
    assert np.array_equal(y1.cpu().numpy()[rows].astype(np.int64), acc)


@pytest.mark.parametrize("bits_w,bits_a,T,N,d", [(3, 3, 200, 256, 4096), (4, 6, 130, 200, 4096), (3, 3, 70, 96, 256),
                                                 (4, 6, 33, 130, 16384), (3, 6, 64, 64, 1024)])
def test_lowbit_layer_small(bits_w, bits_a, T, N, d):
    xf = workloads.small_case(1500 + d, T, d, "t3")
    wf = workloads.small_case(1501 + d, N, d, "w")
    xh, wh = workloads.f32_to_bf16_bits(xf), workloads.f32_to_bf16_bits(wf)
    xf, wf = workloads.bf16_bits_to_f32(xh), workloads.bf16_bits_to_f32(wh)
    seed = 53
    R = rtq.Rpbh.from_seed(seed, d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, bits_a), rtq.Codebook.for_dim(d, bits_w)
    wcodes = torch.empty((N, d * bits_w // 8), dtype=torch.uint8, device="cuda")
    wnorm = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wcodes, wnorm, R, rtq.RTQ_CODEBOOK, cb_w, 0.0)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_CODEBOOK_I8, bits_a), dtype=torch.uint8,
                     device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wcodes, wnorm, y, rtq.RTQ_CODEBOOK_I8, cb_a, cb_w, workspace=ws)
    torch.cuda.synchronize()
    pi = dense_pi(seed, d)
    ocb_a, ocb_w = oracle.lloyd_max(bits_a, d), oracle.lloyd_max(bits_w, d)
    wo = oracle.weights_codebook(wf, pi, ocb_w, bits_w)
    assert codebook_mismatches_allowed(oracle.unpack(wcodes.cpu().numpy(), d, bits_w), wo["codes"], wo["u"],
                                       ocb_w["boundaries"], d)[1] == 0
    out = oracle.qlinear_codebook(xf, pi, wo, ocb_a, ocb_w, bits_a)
    _, ta = int8_table(ocb_a["centroids"])
    a_codes = codes_of(ws[:T * d].view(T, d).cpu().numpy().view(np.int8), ta)
    assert codebook_mismatches_allowed(a_codes, out["act"]["codes"], out["act"]["u"], ocb_a["boundaries"], d)[1] == 0
    got = workloads.bf16_bits_to_f32(bf16_host(y))
    assert rel_fro(got, out["y"]) <= 2e-2


@pytest.mark.parametrize("variant", ["w3a3", "w4a6"])
def test_lowbit_dit_shape_sampled(variant):
    # the benchmark's layers at the attention-output shape (4608 x 4096 -> 4096), full launches;
    # 64 tokens x 256 channels covering every output tile
    ref = dit_cases.codebook_sample(variant)
    d, N, bits_w, bits_a = ref["d"], ref["N"], ref["bits_w"], ref["bits_a"]
    xh, wh = workloads.dit_activations_bf16(d), workloads.w4a4_weight_bf16()
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
    a_codes = codes_of(work[:T * d].view(T, d).cpu().numpy().view(np.int8)[rows], ref["ta"])
    assert codebook_mismatches_allowed(a_codes, ao["codes"], ao["u"], ocb_a["boundaries"], d)[1] == 0
    got = workloads.bf16_bits_to_f32(bf16_host(y))[np.ix_(rows, cols)]
    assert rel_fro(got, ref["y"]) <= 2e-2
    same = np.all(a_codes == ao["codes"], axis=1)[:, None] & np.all(w_codes == wo["codes"], axis=1)[None, :]
    assert same.mean() > 0.9
    assert np.all(bf16_within_one_ulp(got, ref["y_int8"])[same])


def test_split_workspace_shared_across_weight_widths():
    # One workspace reused by products of different weight widths (different kernel variants):
    # the split counters are zeroed before every split launch, so arrivals left by one variant are
    # never read as the current launch's.  Each split product must equal the unsplit one.
    T, N, d = 4608, 4096, 4096          # 288 tiles: shared along d by stream-K runs
    rng = np.random.default_rng(17)
    ws = rtq.new_qgemm_workspace()
    s_a = to_dev(np.ones(T, np.float32))
    s_w = to_dev(np.ones(N, np.float32))
    cb4 = rtq.Codebook.for_dim(d, 4)
    runs = []
    for bits_w in (4, 3, 2, 4, 3, 4):
        qa = to_dev(rng.integers(-127, 128, size=(T, d)).astype(np.int8))
        qw = to_dev(oracle.pack(rng.integers(0, 1 << bits_w, size=(N, d)).astype(np.uint8), bits_w))
        cb_w = rtq.Codebook.for_dim(d, bits_w)
        y0 = torch.empty((T, N), dtype=torch.int32, device="cuda")
        y1 = torch.full((T, N), -1, dtype=torch.int32, device="cuda")
        rtq.qgemm(qa, s_a, qw, s_w, y0, d, rtq.RTQ_CODEBOOK_I8, cb4, cb_w)
        rtq.qgemm(qa, s_a, qw, s_w, y1, d, rtq.RTQ_CODEBOOK_I8, cb4, cb_w, workspace=ws)
        torch.cuda.synchronize()
        runs.append(bool(torch.equal(y0, y1)))
    assert all(runs), runs
