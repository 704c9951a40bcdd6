"""GPU parity of the tiled INT8 format (RTQ_INT8_TILED): the symmetric INT8 codes and scales of
RTQ_INT8 (the rule of "量化旋转主模型是什么？一文读懂低比特图像生成模型", section 4, on the rotated rows
of the OrbitQuant article, sections 2.1-2.2), with the codes stored as the product's 256-row x
64-byte stage blocks.  The layout is undone on the host (tests/_helpers.untile_codes, written from
the layout's definition in include/rtq.h) and the codes compared with the oracle's; products take
tiled operands built on the host from seeded codes and must give the oracle's int64 sums exactly."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
import _dit_cases as dit_cases
from _helpers import bf16_host, dense_pi, int8_mismatches_allowed, tile_codes, to_dev, untile_codes

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
