"""GPU parity of the tiled formats.

RTQ_INT8_TILED: the symmetric INT8 codes and scales of RTQ_INT8 (the rule of
"量化旋转主模型是什么？一文读懂低比特图像生成模型", section 4, on the rotated rows of the OrbitQuant
article, sections 2.1-2.2), with the codes stored as the product's 256-row x 64-byte stage blocks.
RTQ_CODEBOOK_TILED / RTQ_CODEBOOK_I8_TILED: the Lloyd-Max codes of the OrbitQuant article
(sections 1, 2.1-2.2, 4.2), weights as packed codes in the tiled code layout and activations as
int8 codebook values in the INT8 tiled layout.

The layouts are undone on the host (tests/_helpers.untile_codes / untile_packed, written from the
layouts' definitions in include/rtq.h and pinned to them by a CPU test) and the codes compared
with the oracle's and with the row-major modes'; products take tiled operands built on the host
from seeded codes and must give the oracle's int64 sums exactly."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
import _dit_cases as dit_cases
from _helpers import (bf16_host, codebook_mismatches_allowed, codes_of, dense_pi, int8_mismatches_allowed,
                      int8_table, rel_fro, tile_codes, tile_packed, to_dev, untile_codes, untile_packed)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


@pytest.mark.parametrize("rows,d,xt", [(300, 256, "f32"), (513, 1024, "bf16"), (257, 4096, "bf16"),
                                       (70, 16384, "bf16"), (256, 4096, "bf16"), (33, 64, "bf16")])
def test_quantize_tiled_matches_oracle(rows, d, xt):
    seed = 81
    xf = workloads.small_case(8100 + d + rows, rows, d, "t3")
    if xt == "bf16":
        xh = workloads.f32_to_bf16_bits(xf)
        xf = workloads.bf16_bits_to_f32(xh)
        xd = to_dev(xh, "bf16")
    else:
        xd = to_dev(xf)
    R = rtq.Rpbh.from_seed(seed, d)
    codes = torch.zeros(rtq.tiled_rows(rows) * d, dtype=torch.int8, device="cuda")
    scale = torch.empty(rows, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(xd, codes, scale, R, rtq.RTQ_INT8_TILED)
    flat = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    scale_flat = torch.empty(rows, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(xd, flat, scale_flat, R, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    got = untile_codes(codes.cpu().numpy(), rows, d)
    wo = oracle.weights_int8(xf, dense_pi(seed, d), True)
    assert np.array_equal(workloads.bf16_bits_to_f32(bf16_host(scale)), wo["scale"])
    assert int8_mismatches_allowed(got, wo["q"], wo["pre"])[1] == 0
    # the same codes as the row-major format, and padding rows untouched
    assert np.array_equal(got, flat.cpu().numpy())
    assert torch.equal(scale.view(torch.int16), scale_flat.view(torch.int16))
    full = untile_codes(codes.cpu().numpy(), rtq.tiled_rows(rows), d)
    assert not full[rows:].any()


@pytest.mark.parametrize("T,N,d,ws", [(130, 200, 256, False), (300, 700, 2048, True), (4100, 4100, 1024, True),
                                      (4608, 4096, 4096, True), (257, 129, 64, False)])
def test_tiled_product_accumulators_bit_exact(T, N, d, ws):
    # raw int32 sums against the oracle's int64 product; with the workspace, a partial last round
    # is shared along d (split ranges, or stream-K runs for 289 and 288 tiles)
    rng = np.random.default_rng(T + N + d)
    a = rng.integers(-127, 128, size=(T, d)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, d)).astype(np.int8)
    rows = np.arange(T) if T * N <= 1 << 18 else np.sort(rng.choice(T, 48, replace=False))
    ref = oracle.gemm_int8(a[rows], w)
    acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
    work = rtq.new_qgemm_workspace() if ws else None
    rtq.qgemm(to_dev(tile_codes(a)), to_dev(np.ones(T, np.float32)), to_dev(tile_codes(w)),
              to_dev(np.ones(N, np.float32)), acc, d, rtq.RTQ_INT8_TILED, workspace=work, n_tokens=T, n_out=N)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), ref)


def test_tiled_layer_dit_shape_matches_row_major_and_oracle():
    # the benchmark's W8A8 DiT layer (4608 x 4096 -> 16384) in both formats: the same codes and the
    # same exact sums, so the outputs agree bit for bit; 64 tokens x 256 channels covering every
    # output tile against the oracle, element by element within one bf16 ulp
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh, wh = workloads.dit_activations_bf16(d), workloads.dit_weight_bf16("mlp_up")
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    w_dev, x_dev = to_dev(wh, "bf16"), to_dev(xh, "bf16")
    wq_t = torch.empty(rtq.tiled_rows(N) * d, dtype=torch.int8, device="cuda")
    ws_t = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(w_dev, wq_t, ws_t, R, rtq.RTQ_INT8_TILED)
    wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
    ws = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(w_dev, wq, ws, R, rtq.RTQ_INT8)
    y_t = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_INT8_TILED), dtype=torch.uint8, device="cuda")
    rtq.rotated_qlinear(x_dev, R, wq_t, ws_t, y_t, rtq.RTQ_INT8_TILED, workspace=work)
    rtq.rotated_qlinear(x_dev, R, wq, ws, y)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y.view(torch.int16))
    ref = dit_cases.w8a8_sample()
    rows, cols = ref["rows"], ref["cols"]
    w_codes = untile_codes(wq_t.cpu().numpy(), N, d)[cols]
    assert int8_mismatches_allowed(w_codes, ref["wo"]["q"], ref["wo"]["pre"])[1] == 0
    a_codes = untile_codes(work[:rtq.tiled_rows(T) * d].cpu().numpy(), T, d)[rows]
    assert int8_mismatches_allowed(a_codes, ref["ao"]["q"], ref["ao"]["pre"])[1] == 0
    off = rtq.tiled_rows(T) * d
    assert np.array_equal(work[off:off + 4 * T].view(torch.float32).cpu().numpy()[rows], ref["ao"]["scale"])
    got = workloads.bf16_bits_to_f32(bf16_host(y_t))[np.ix_(rows, cols)]
    same = (np.all(a_codes == ref["ao"]["q"], axis=1)[:, None] & np.all(w_codes == ref["wo"]["q"], axis=1)[None, :])
    assert same.mean() > 0.9
    assert np.all(dit_cases.bf16_within_one_ulp(got, ref["y"])[same])


def test_tiled_small_layer_fp32():
    # the tiny fp32 layer (d_in 256 -> 512, 128 tokens) in the tiled format: fp32 output within 1e-4
    inp = workloads.tiny_inputs()
    x, w = inp["x"], inp["w"]
    d = 256
    R = rtq.Rpbh.from_seed(inp["rpbh_seed"], d)
    wq = torch.empty(rtq.tiled_rows(512) * d, dtype=torch.int8, device="cuda")
    ws = torch.empty(512, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(w), wq, ws, R, rtq.RTQ_INT8_TILED)
    y = torch.empty((128, 512), dtype=torch.float32, device="cuda")
    rtq.rotated_qlinear(to_dev(x), R, wq, ws, y, rtq.RTQ_INT8_TILED)
    torch.cuda.synchronize()
    pi = dense_pi(inp["rpbh_seed"], d)
    ref = oracle.qlinear_int8(x, pi, oracle.weights_int8(w, pi, False))["y"]
    got = y.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-4


def _rows_input(rows, d, xt, seed):
    xf = workloads.small_case(seed, rows, d, "t3")
    if xt == "bf16":
        xh = workloads.f32_to_bf16_bits(xf)
        return workloads.bf16_bits_to_f32(xh), to_dev(xh, "bf16")
    return xf, to_dev(xf)


@pytest.mark.parametrize("rows,d,bits,xt,rot", [(300, 256, 4, "bf16", True), (513, 1024, 2, "bf16", True),
                                                (257, 4096, 3, "bf16", True), (70, 16384, 2, "bf16", True),
                                                (256, 4096, 4, "bf16", True), (33, 512, 4, "f32", False),
                                                (130, 256, 2, "f32", True)])
def test_quantize_codebook_tiled_weights(rows, d, bits, xt, rot):
    # the weight form (bf16 norms, eps = 0) in the tiled code layout: the row-major mode's bytes,
    # the oracle's codes up to the boundary allowance, padding rows untouched
    xf, xd = _rows_input(rows, d, xt, 8200 + d + rows)
    seed = 83
    R = rtq.Rpbh.from_seed(seed, d) if rot else None
    cb = rtq.Codebook.for_dim(d, bits)
    codes_t = torch.zeros(rtq.tiled_code_bytes(rows, d, rtq.RTQ_CODEBOOK_TILED, bits), dtype=torch.uint8, device="cuda")
    s_t = torch.empty(rows, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(xd, codes_t, s_t, R, rtq.RTQ_CODEBOOK_TILED, cb, 0.0)
    codes = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(xd, codes, s, R, rtq.RTQ_CODEBOOK, cb, 0.0)
    torch.cuda.synchronize()
    buf = codes_t.cpu().numpy()
    got = untile_packed(buf, rows, d, bits)
    assert np.array_equal(got, codes.cpu().numpy())
    assert torch.equal(s_t.view(torch.int16), s.view(torch.int16))
    assert not untile_packed(buf, rtq.tiled_rows(rows), d, bits)[rows:].any()
    ocb = oracle.lloyd_max(bits, d)
    v = oracle.rotate(xf, dense_pi(seed, d))[1] if rot else xf
    co, so, u = oracle.quantize_codebook(v, ocb["boundaries"], True, 0.0)
    assert np.array_equal(workloads.bf16_bits_to_f32(bf16_host(s_t)), so)
    assert codebook_mismatches_allowed(oracle.unpack(got, d, bits), co, u, ocb["boundaries"], d)[1] == 0


@pytest.mark.parametrize("rows,d,bits,xt,rot", [(300, 256, 4, "bf16", True), (513, 1024, 2, "bf16", True),
                                                (257, 4096, 3, "bf16", True), (70, 16384, 4, "bf16", True),
                                                (130, 4096, 6, "bf16", True), (33, 512, 4, "f32", False)])
def test_quantize_codebook_i8_tiled_activations(rows, d, bits, xt, rot):
    # the activation form (fp32 norms, eps = 1e-8) as int8 codebook values in the INT8 tiled layout
    xf, xd = _rows_input(rows, d, xt, 8300 + d + rows)
    seed = 84
    R = rtq.Rpbh.from_seed(seed, d) if rot else None
    cb = rtq.Codebook.for_dim(d, bits)
    vals_t = torch.zeros(rtq.tiled_rows(rows) * d, dtype=torch.int8, device="cuda")
    s_t = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(xd, vals_t, s_t, R, rtq.RTQ_CODEBOOK_I8_TILED, cb, 1e-8)
    vals = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(xd, vals, s, R, rtq.RTQ_CODEBOOK_I8, cb, 1e-8)
    torch.cuda.synchronize()
    buf = vals_t.cpu().numpy()
    got = untile_codes(buf, rows, d)
    assert np.array_equal(got, vals.cpu().numpy())
    assert torch.equal(s_t, s)
    assert not untile_codes(buf, rtq.tiled_rows(rows), d)[rows:].any()
    ocb = oracle.lloyd_max(bits, d)
    _, table = int8_table(ocb["centroids"])
    v = oracle.rotate(xf, dense_pi(seed, d))[1] if rot else xf
    co, so, u = oracle.quantize_codebook(v, ocb["boundaries"], False, 1e-8)
    assert np.array_equal(s_t.cpu().numpy(), so)
    assert codebook_mismatches_allowed(codes_of(got, table), co, u, ocb["boundaries"], d)[1] == 0


@pytest.mark.parametrize("T,N,d,bits_w,ws", [(130, 200, 256, 4, False), (300, 700, 2048, 2, True),
                                             (4100, 4100, 1024, 4, True), (4608, 4096, 4096, 4, True),
                                             (257, 129, 64, 3, False), (600, 520, 1024, 3, True),
                                             (1000, 300, 4096, 2, True)])
def test_tiled_codebook_product_accumulators_bit_exact(T, N, d, bits_w, ws):
    # raw int32 sums of int8 activation values times the weight codes' int8 values, both operands
    # tiled, against the oracle's int64 product of the same tables (fp32 table rule of the mode)
    rng = np.random.default_rng(T + N + d + bits_w)
    ocb_a, ocb_w = oracle.lloyd_max(4, d), oracle.lloyd_max(bits_w, d)
    _, ta = int8_table(ocb_a["centroids"])
    _, tw = int8_table(ocb_w["centroids"])
    a = ta[rng.integers(0, 16, size=(T, d), dtype=np.uint8)].astype(np.int8)
    cw = rng.integers(0, 1 << bits_w, size=(N, d), dtype=np.uint8)
    rows = np.arange(T) if T * N <= 1 << 18 else np.sort(rng.choice(T, 48, replace=False))
    ref = oracle.gemm_int8(a[rows], tw[cw].astype(np.int8))
    acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
    work = rtq.new_qgemm_workspace() if ws else None
    cba, cbw = rtq.Codebook.for_dim(d, 4), rtq.Codebook.for_dim(d, bits_w)
    print(f"tiled codebook product T={T} N={N} d={d} bits_w={bits_w} ws={ws}", flush=True)
    rtq.qgemm(to_dev(tile_codes(a)), to_dev(np.ones(T, np.float32)), to_dev(tile_packed(oracle.pack(cw, bits_w), bits_w)),
              to_dev(np.ones(N, np.float32)), acc, d, rtq.RTQ_CODEBOOK_I8_TILED, cba, cbw, workspace=work,
              n_tokens=T, n_out=N)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), ref)


@pytest.mark.parametrize("variant", ["w4a4", "w2a4", "w3a3", "w4a6"])
def test_tiled_codebook_layer_dit_shape(variant):
    # the benchmark's codebook layers in both layouts: the same codes and the same exact sums, so
    # the outputs agree bit for bit; 64 tokens x 256 channels covering every output tile against
    # the oracle (the row-major layer's bar: 2e-2 relative Frobenius against the exact-centroid
    # product, one bf16 ulp against the same codes through the int8 tables)
    d, N, bits_w, bits_a, wgen = dit_cases.CODEBOOK_VARIANTS[variant]
    xh, wh = workloads.dit_activations_bf16(d), wgen()
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, bits_a), rtq.Codebook.for_dim(d, bits_w)
    print(f"tiled codebook layer {variant}: {T} x {d} -> {N}", flush=True)
    w_dev, x_dev = to_dev(wh, "bf16"), to_dev(xh, "bf16")
    wct = torch.empty(rtq.tiled_code_bytes(N, d, rtq.RTQ_CODEBOOK_TILED, bits_w), dtype=torch.uint8, device="cuda")
    wnt = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(w_dev, wct, wnt, R, rtq.RTQ_CODEBOOK_TILED, cb_w, 0.0)
    wc = torch.empty((N, d * bits_w // 8), dtype=torch.uint8, device="cuda")
    wn = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(w_dev, wc, wn, R, rtq.RTQ_CODEBOOK, cb_w, 0.0)
    y_t = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_CODEBOOK_I8_TILED, bits_a), dtype=torch.uint8,
                       device="cuda")
    rtq.rotated_qlinear(x_dev, R, wct, wnt, y_t, rtq.RTQ_CODEBOOK_I8_TILED, cb_a, cb_w, workspace=work)
    rtq.rotated_qlinear(x_dev, R, wc, wn, y, rtq.RTQ_CODEBOOK_I8, cb_a, cb_w)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y.view(torch.int16))
    assert np.array_equal(untile_packed(wct.cpu().numpy(), N, d, bits_w), wc.cpu().numpy())
    ref = dit_cases.codebook_sample(variant)
    rows, cols, wo, ao = ref["rows"], ref["cols"], ref["wo"], ref["ao"]
    ocb_a, ocb_w = ref["ocb_a"], ref["ocb_w"]
    w_codes = oracle.unpack(wc.cpu().numpy()[cols], d, bits_w)
    assert codebook_mismatches_allowed(w_codes, wo["codes"], wo["u"], ocb_w["boundaries"], d)[1] == 0
    a_codes = codes_of(untile_codes(work[:rtq.tiled_rows(T) * d].cpu().numpy(), T, d)[rows], ref["ta"])
    assert codebook_mismatches_allowed(a_codes, ao["codes"], ao["u"], ocb_a["boundaries"], d)[1] == 0
    off = rtq.tiled_rows(T) * d
    assert np.array_equal(work[off:off + 4 * T].view(torch.float32).cpu().numpy()[rows], ao["norm"])
    got = workloads.bf16_bits_to_f32(bf16_host(y_t))[np.ix_(rows, cols)]
    assert rel_fro(got, ref["y"]) <= 2e-2
    same = np.all(a_codes == ao["codes"], axis=1)[:, None] & np.all(w_codes == wo["codes"], axis=1)[None, :]
    assert same.mean() > 0.9
    assert np.all(dit_cases.bf16_within_one_ulp(got, ref["y_int8"])[same])
